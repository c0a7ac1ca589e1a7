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

// Hot-path class record kept in LDS by the fused kernels (96 bytes, six 16-byte rows).
// The absolute values of a class are unranked in at most two parts.  Odd classes and
// even classes with w = 0 or w = 24 have one part of 24 values; other even classes have
// the support part (w values, placed on the codeword's positions) followed by the
// complement part (24 - w values).  Per part X (0 = first, 1 = second):
//   ncX  SWAR thresholds: byte j-1 (j = 1..3) = 0x80 - C_j, C_j = sum of the counts of
//        value slots below j; unused slots have count 0.
//   cntX counts of the part's value slots 0..3 times 8, one per byte (8 c_j <= 192: the
//        byte is the offset of entry c_j in a row of 8-byte table entries).
//   svX  8-byte table read with v_perm (svXhi:svXlo), entries biased by +12:
//        even classes: bytes 0-3 = 12 + |v_j|, bytes 4-7 = 12 - |v_j| (negative sign);
//        odd classes:  bytes 0-3 = 12 + b(v_j) for positions on the codeword,
//                      bytes 4-7 = 12 - b(v_j) off it, b(v) = v if v = 1 mod 4 else -v.
//   svX8 the same 8-byte table with signed values as OCP fp8 E4M3 codes (exact for |v| <= 12;
//        zero as 0x00), read by the batch-1 GEMV, which converts value pairs to bf16.
// meta: B (bits 0-4) | w (bits 8-12) | pi (bit 16) | parity (bit 17) |
//       nonzero mask of part-0 slots (bits 20-23) | nonzero mask of part-1 slots (24-27).
struct LlvqClassHot {
  double start;      // first global index (exact in fp64)
  double y0s;        // n0 / P: length of the first part over the number of arrangements
  double inv_a;      // 1 / A
  double a;          // A
  uint32_t toff;     // Golay table position of codeword r = 0
  uint32_t meta;
  float invnorm;     // fp32 1/(4 sqrt m), computed in fp64 and rounded once
  uint32_t m;        // shell
  uint32_t nc0, cnt0, sv0lo, sv0hi;   // part 0 (byte offset 48)
  uint32_t nc1, cnt1, sv1lo, sv1hi;   // part 1 (byte offset 64: one 16-byte read)
  uint32_t sv0lo8, sv0hi8, sv1lo8, sv1hi8;   // fp8 tables of parts 0 and 1 (byte offset 80)
};

// Composition record of a tail table of the last n = 6 or 7 positions (see gen_tables.cpp).
struct LlvqTailComp {
  float q_over_n;    // arrangements of the composition / n (n = 6 or 7 tail positions)
  uint32_t offset;   // first entry of the composition's group in the tail table
};

// Class record of the rank (point -> index) kernel.
struct LlvqClassRank {
  uint64_t start;    // first global shape index of the class
  double p_s;        // arrangements of the support values (even classes; 1 for odd)
  double p_t;        // arrangements of the complement values (odd classes: all 24 values)
  uint32_t A;        // codewords the index r ranges over
  uint32_t toff;     // position in the sorted Golay table of codeword r = 0
  uint32_t key;      // s1 | s3 << 6 | s4 << 17, s_k = sum of |x_i|^k
  uint32_t slot_lo;  // slot of absolute value a in its part, byte (a >> 1), a >> 1 = 0..3
  uint32_t slot_hi;  //   ... a >> 1 = 4..7; 0x80 = value not in the class
  uint32_t cnt_s;    // counts of the support slots (even classes), one per byte
  uint32_t cnt_t;    // counts of the complement slots (odd classes: all values)
  uint32_t meta;     // B | w << 8 | pi << 16 | parity << 17 | m << 20
};

// Class record of the general decoder (shells 2..42; gen_tables --wide).  Inside a class
// every quantity fits 64 bits; the global start needs 128.
struct LlvqWideClass {
  uint64_t start_lo, start_hi;   // first global shape index
  uint64_t P_S;                  // arrangements of the support values (even classes; 1 for odd)
  uint64_t P_T;                  // arrangements of the complement values (odd classes: all 24)
  uint8_t m, parity, w, B, pi;   // shell, coset, support length, sign bits, support sign parity
  uint8_t nsup, ncomp, pad;      // distinct support / complement values
  uint8_t sv[8], sc[8];          // support multiset: distinct values ascending, their counts
  uint8_t cv[8], cc[8];          // complement multiset (odd classes: all 24 values)
};
