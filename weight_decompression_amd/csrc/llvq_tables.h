// Table record layout shared by the generated table header and the HIP library.
#pragma once
#include <stdint.h>

// One class of the shell union (a leader multiset together with its even or odd
// coset).  Field order matches the initialisers written by gen_tables.cpp.
struct LlvqClassRec {
  uint64_t start;    // first global shape index of the class
  double inv_p;      // 1 / P with P = P_S * P_T arrangements of the absolute values
  uint32_t A;        // codewords the index r ranges over: 1, 759, 2576 or 4096
  uint32_t toff;     // position in the sorted Golay table of codeword r = 0
  uint32_t vals_s;   // even: distinct support values (= 2 mod 4), ascending, one per byte
  uint32_t cnt_s;    //       their multiplicities
  uint32_t vals_t;   // even: distinct complement values (= 0 mod 4); odd: all values
  uint32_t cnt_t;    //       their multiplicities
  uint32_t p_t;      // arrangements of the complement values
  uint8_t B;         // sign bits
  uint8_t parity;    // 0 even coset, 1 odd coset
  uint8_t pi;        // even: parity of the number of negative support entries
  uint8_t m;         // shell
  uint8_t w;         // even: support length (codeword weight); odd: 0
  uint8_t d_s;       // distinct support values
  uint8_t d_t;       // distinct complement values
  uint8_t pad;
};
