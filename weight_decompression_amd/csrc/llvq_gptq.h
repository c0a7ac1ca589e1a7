// Spherical GPTQ on the GPU (gfx950), fp64: the inverse-Hessian factor and the per-block-
// column error feedback ("LLVQ", papernotes.org notes, 关键设计 3: shape-gain quantisation
// with GPTQ's curvature compensation; a block's lattice direction is rescaled to the block's
// own norm, a retraction onto the product of spheres, and the residual is spread over the
// columns not yet quantised through U = chol(H^-1)^T).  Included once by llvq.hip.
//
// Factor.  H is padded to Kp = 24 Kb columns (pad columns: an uncoupled diagonal equal to the
// mean of diag H) and damped, Hd = Hp + damp mean(diag H) I.  With P the index reversal,
// P Hd P = M M^T (M lower, Cholesky) gives Hd = V V^T with V = P M P upper, so
// Hd^-1 = (V^-1)^T V^-1 and U = V^-1 = P M^-1 P: a Cholesky factorisation and a triangular
// inverse of the reversed matrix, no explicit inverse of Hd.  Both are blocked by 24:
//   Cholesky, block step j: factor the diagonal block (and invert it), solve the panel below
//     it, update the trailing lower triangle (one launch each);
//   inverse, block row i: X_ij = -Linv_ii sum_{j <= k < i} L_ik X_kj for every j < i (one
//     launch per block row; the blocks of earlier rows are final).
// Then U is X with both indices reversed (in place).
//
// Column step b (S = columns 24b .. 24b + 23, F = the columns after S), every row r:
//   v = the angular nearest point chosen by the search kernel for W[r, S];
//   nrm = |W[r, S]|, g = the gain table entry nearest to nrm (ties to the lower index);
//   w_hat = nrm v / |v| (spherical) or G[g] v / |v| (Euclidean feedback);
//   E = W[r, S] - w_hat, E' = E U_SS^-1 (a 24 x 24 triangular solve);
//   W[r, F] -= E' U_SF, and the next block column goes out as fp32 for the next search.
// The order of every fp64 sum is fixed, so results do not depend on the launch.

#pragma once

constexpr int kGB = 24;                 // block size of the factorisation = the LLVQ block
constexpr int kGTile = 64;              // trailing-update tile (64 x 64, 16 outputs per lane)

// ---------------------------------------------------------------------------
// factor

// mean of diag H (one workgroup, fixed-order reduction)
__global__ __launch_bounds__(256) void k_gptq_diag_mean(const double* __restrict__ H, int K, double* __restrict__ mean) {
  __shared__ double part[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < K; i += 256) s += H[(size_t)i * (size_t)K + (size_t)i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) mean[0] = part[0] / (double)K;
}

// A = P Hd P over Kp x Kp: A[i][j] = Hd[Kp-1-i][Kp-1-j]
__global__ __launch_bounds__(256) void k_gptq_reverse_damp(const double* __restrict__ H, int K, int Kp,
                                                           const double* __restrict__ mean, double damp,
                                                           double* __restrict__ A) {
  const size_t n = (size_t)Kp * (size_t)Kp;
  const double mu = mean[0];
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) {
    const int i = (int)(e / (size_t)Kp), j = (int)(e - (size_t)i * (size_t)Kp);
    const int si = Kp - 1 - i, sj = Kp - 1 - j;
    double h;
    if (si < K && sj < K)
      h = H[(size_t)si * (size_t)K + (size_t)sj];
    else
      h = si == sj ? mu : 0.0;
    if (si == sj) h += damp * mu;
    A[e] = h;
  }
}

// Cholesky of the 24 x 24 diagonal block at j0 (in place, lower) and its inverse into
// Linv[jb] (24 x 24, lower, row-major).  One workgroup of 64 lanes.
__global__ __launch_bounds__(64) void k_gptq_potrf_diag(double* __restrict__ A, int Kp, int j0,
                                                        double* __restrict__ Linv, int* __restrict__ bad) {
  __shared__ double a[kGB][kGB + 1];
  __shared__ double li[kGB][kGB + 1];
  const int t = threadIdx.x;
  // lane t < 24 holds row t of the block in registers; the pivot and column k reach the
  // other lanes by wave shuffles (one wave: no barrier inside the factorisation)
  double row[kGB];
#pragma unroll
  for (int c = 0; c < kGB; ++c) row[c] = t < kGB ? A[(size_t)(j0 + t) * Kp + (size_t)(j0 + c)] : 0.0;
#pragma unroll
  for (int k = 0; k < kGB; ++k) {
    const double d = __shfl(row[k], k, 64);               // a[k][k]
    if (t == 0 && !(d > 0.0) && bad) atomicAdd(bad, 1);
    const double akk = d > 0.0 ? sqrt(d) : 1.0;
    if (t == k) row[k] = akk;
    if (t > k && t < kGB) row[k] /= akk;
    // rank-1 update of the rest of the block (lower part): a[t][c] -= a[t][k] a[c][k]
#pragma unroll
    for (int c = k + 1; c < kGB; ++c) {
      const double ack = __shfl(row[k], c, 64);           // a[c][k], divided
      if (t >= c && t < kGB) row[c] -= row[k] * ack;
    }
  }
  if (t < kGB) {
#pragma unroll
    for (int c = 0; c < kGB; ++c) a[t][c] = row[c];
  }
  __syncthreads();
  // inverse of the lower factor, column by column (forward substitution; lane c owns column
  // c and keeps it in registers; the rows of the factor are LDS broadcasts)
  if (t < kGB) {
    double lc[kGB];
#pragma unroll
    for (int r = 0; r < kGB; ++r) {
      double s = (r == t) ? 1.0 : 0.0;
#pragma unroll
      for (int q = 0; q < r; ++q)
        if (q >= t) s -= a[r][q] * lc[q];
      lc[r] = r < t ? 0.0 : s / a[r][r];
    }
#pragma unroll
    for (int r = 0; r < kGB; ++r) li[r][t] = lc[r];
  }
  __syncthreads();
  for (int e = t; e < kGB * kGB; e += 64) {
    const int r = e / kGB, c = e % kGB;
    A[(size_t)(j0 + r) * Kp + (size_t)(j0 + c)] = c <= r ? a[r][c] : 0.0;
    Linv[e] = li[r][c];
  }
}

// panel below the diagonal block: A[i][j0..j0+23] <- A[i][j0..] Linv_jj^T for i >= j0 + 24
__global__ __launch_bounds__(256) void k_gptq_panel(double* __restrict__ A, int Kp, int j0,
                                                    const double* __restrict__ Linv) {
  __shared__ double li[kGB * kGB];
  for (int e = threadIdx.x; e < kGB * kGB; e += 256) li[e] = Linv[e];
  __syncthreads();
  const int i = j0 + kGB + blockIdx.x * 256 + threadIdx.x;
  if (i >= Kp) return;
  double* row = A + (size_t)i * Kp + (size_t)j0;
  double x[kGB];
#pragma unroll
  for (int c = 0; c < kGB; ++c) x[c] = row[c];
#pragma unroll
  for (int c = 0; c < kGB; ++c) {
    double s = 0.0;
#pragma unroll
    for (int q = 0; q <= c; ++q) s = fma(x[q], li[c * kGB + q], s);
    row[c] = s;
  }
}

// trailing update of the lower triangle: A[i][i2] -= sum_q A[i][j0+q] A[i2][j0+q] for
// i >= i2 >= j0 + 24; 64 x 64 tiles (lower tiles only), 16 outputs per lane.
__global__ __launch_bounds__(256) void k_gptq_syrk(double* __restrict__ A, int Kp, int j0) {
  const int ti = blockIdx.y, tj = blockIdx.x;
  if (tj > ti) return;
  const int base = j0 + kGB;
  const int r0 = base + ti * kGTile, c0 = base + tj * kGTile;
  __shared__ double pr[kGTile][kGB + 1];
  __shared__ double pc[kGTile][kGB + 1];
  for (int e = threadIdx.x; e < kGTile * kGB; e += 256) {
    const int r = e / kGB, q = e % kGB;
    pr[r][q] = r0 + r < Kp ? A[(size_t)(r0 + r) * Kp + (size_t)(j0 + q)] : 0.0;
    pc[r][q] = c0 + r < Kp ? A[(size_t)(c0 + r) * Kp + (size_t)(j0 + q)] : 0.0;
  }
  __syncthreads();
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;   // rows tr, tr+16, ...; cols tc, tc+16, ...
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
#pragma unroll 4
  for (int q = 0; q < kGB; ++q) {
    double x[4], yv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) x[a] = pr[tr + 16 * a][q];
#pragma unroll
    for (int b = 0; b < 4; ++b) yv[b] = pc[tc + 16 * b][q];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = fma(x[a], yv[b], acc[a][b]);
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = r0 + tr + 16 * a, i2 = c0 + tc + 16 * b;
      if (i < Kp && i2 <= i) A[(size_t)i * Kp + (size_t)i2] -= acc[a][b];
    }
}

// The triangular inverse X = L^-1 (L = the factor in A) below the diagonal, right-looking:
// block (i, j) first accumulates T_ij = sum_{j <= k < i} L_ik X_kj in place, one k per
// step, and step i finishes it as X_ij = -Linv_ii T_ij.  Per step k two launches, each
// spread over the whole chip (a column-by-column forward substitution would leave the first
// column's ~nb^2/2 block products to one CU):
//   k_gptq_inv_update(k): T_ij += L_ik X_kj for every i > k and j <= k (one workgroup per
//     block, one lane per element; X_kk = Linv_kk, X_kj for j < k finished by the solve of
//     step k), the first term (k = j) starting from 0;
//   k_gptq_inv_solve(k + 1): X_{k+1, j} = -Linv_{k+1} T_{k+1, j} for every j <= k.
// Every element is summed over k, then q, in ascending order (a partial sum T is stored
// between steps exactly, in fp64).
__global__ __launch_bounds__(576) void k_gptq_inv_update(const double* __restrict__ A, int Kp, int kb, double* X) {
  const int ib = kb + 1 + (int)blockIdx.x, jb = (int)blockIdx.y;     // i > k, j <= k
  const int r = threadIdx.x / kGB, c = threadIdx.x % kGB;
  __shared__ double lt[kGB][kGB + 1];
  __shared__ double xt[kGB][kGB + 1];
  const size_t i0 = (size_t)ib * kGB, j0 = (size_t)jb * kGB, k0 = (size_t)kb * kGB;
  double* t = X + (i0 + (size_t)r) * Kp + j0 + (size_t)c;
  double s = jb == kb ? 0.0 : *t;
  lt[r][c] = A[(i0 + (size_t)r) * Kp + k0 + (size_t)c];               // L_ik
  xt[r][c] = X[(k0 + (size_t)r) * Kp + j0 + (size_t)c];               // X_kj
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kGB; ++q) s = fma(lt[r][q], xt[q][c], s);
  *t = s;
}

__global__ __launch_bounds__(576) void k_gptq_inv_solve(int Kp, int ib, const double* __restrict__ Linv, double* X) {
  const int jb = (int)blockIdx.x;           // < ib
  const int r = threadIdx.x / kGB, c = threadIdx.x % kGB;
  __shared__ double ld[kGB][kGB + 1];
  __shared__ double td[kGB][kGB + 1];
  double* t = X + ((size_t)ib * kGB + (size_t)r) * Kp + (size_t)jb * kGB + (size_t)c;
  ld[r][c] = Linv[(size_t)ib * kGB * kGB + threadIdx.x];
  td[r][c] = *t;
  __syncthreads();
  double x = 0.0;
  for (int q = 0; q <= r; ++q) x = fma(ld[r][q], td[q][c], x);
  *t = -x;
}

// diagonal blocks of X (= Linv) and zeros above the diagonal
__global__ __launch_bounds__(256) void k_gptq_inv_diag(int Kp, const double* __restrict__ Linv, double* __restrict__ X) {
  const size_t n = (size_t)Kp * (size_t)Kp;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) {
    const int i = (int)(e / (size_t)Kp), j = (int)(e - (size_t)i * (size_t)Kp);
    if (j > i) {
      X[e] = 0.0;
    } else if (i / kGB == j / kGB) {
      X[e] = Linv[(size_t)(i / kGB) * kGB * kGB + (size_t)(i % kGB) * kGB + (size_t)(j % kGB)];
    }
  }
}

// U = P X P in place: swap every element with its mirror (i, j) <-> (Kp-1-i, Kp-1-j)
__global__ __launch_bounds__(256) void k_gptq_reverse(int Kp, double* __restrict__ X) {
  const size_t n = (size_t)Kp * (size_t)Kp;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n / 2; e += (size_t)gridDim.x * 256) {
    const size_t m = n - 1 - e;
    const double t = X[e];
    X[e] = X[m];
    X[m] = t;
  }
}

// ---------------------------------------------------------------------------
// column steps

// Wq = W (fp32 [rows][cols]) as fp64 [rows][Kp], zero padded; x0 = block column 0 as fp32
__global__ __launch_bounds__(256) void k_gptq_begin(const float* __restrict__ W, int rows, int cols, int Kp,
                                                    double* __restrict__ Wq, float* __restrict__ x0) {
  const size_t n = (size_t)rows * (size_t)Kp;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) {
    const int r = (int)(e / (size_t)Kp), c = (int)(e - (size_t)r * (size_t)Kp);
    const double v = c < cols ? (double)W[(size_t)r * (size_t)cols + (size_t)c] : 0.0;
    Wq[e] = v;
    if (c < kGB) x0[(size_t)r * kGB + (size_t)c] = (float)v;
  }
}

struct GptqCol {
  int rows, Kp, kb, block, variant, gain_bits, shape_bits, last;
};

// one row per lane: nearest gain, retraction, residual E and E' = E U_SS^-1 (into ework
// [rows][24]), and the block's field
__global__ __launch_bounds__(256) void k_gptq_residual(GptqCol g, const double* __restrict__ Wq,
                                                       const double* __restrict__ U, const __half* __restrict__ gains,
                                                       const int8_t* __restrict__ points,
                                                       const uint64_t* __restrict__ indices,
                                                       uint64_t* __restrict__ fields, double* __restrict__ ework) {
  __shared__ double us[kGB][kGB + 1];
  __shared__ double G[256];
  const int s0 = g.block * kGB;
  for (int e = threadIdx.x; e < kGB * kGB; e += 256)
    us[e / kGB][e % kGB] = U[(size_t)(s0 + e / kGB) * g.Kp + (size_t)(s0 + e % kGB)];
  for (int e = threadIdx.x; e < (1 << g.gain_bits); e += 256) G[e] = (double)__half2float(gains[e]);
  __syncthreads();
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= g.rows) return;
  const double* w = Wq + (size_t)r * g.Kp + (size_t)s0;
  double wv[kGB], vv[kGB];
  double n2 = 0.0, v2 = 0.0;
#pragma unroll
  for (int c = 0; c < kGB; ++c) {
    wv[c] = w[c];
    vv[c] = (double)points[(size_t)r * kGB + (size_t)c];
    n2 = fma(wv[c], wv[c], n2);
    v2 = fma(vv[c], vv[c], v2);
  }
  const double nrm = sqrt(n2);
  // nearest gain (ties to the lower index)
  int gi = 0;
  double best = fabs(G[0] - nrm);
  for (int e = 1; e < (1 << g.gain_bits); ++e) {
    const double d = fabs(G[e] - nrm);
    if (d < best) {
      best = d;
      gi = e;
    }
  }
  fields[(size_t)r * g.kb + (size_t)g.block] = indices[r] | ((uint64_t)gi << g.shape_bits);
  if (g.variant == 2 || g.last) return;       // direct quantisation, or no columns left
  const double vn = sqrt(v2);
  const double len = g.variant == 1 ? G[gi] : nrm;
  double e[kGB];
#pragma unroll
  for (int c = 0; c < kGB; ++c) e[c] = wv[c] - len * (vv[c] / vn);
  // E' U_SS = E: forward substitution over the columns of the upper triangular U_SS
  double* eo = ework + (size_t)r * kGB;
#pragma unroll
  for (int c = 0; c < kGB; ++c) {
    double s = e[c];
#pragma unroll
    for (int q = 0; q < c; ++q) s = fma(-e[q], us[q][c], s);
    e[c] = s / us[c][c];
    eo[c] = e[c];
  }
}

// W[r][F] -= E'[r] U_SF, 32 rows x 256 columns per workgroup (one column per lane, its 24 U
// values in registers); the next block column's final values also go out as fp32
__global__ __launch_bounds__(256) void k_gptq_update(GptqCol g, double* __restrict__ Wq, const double* __restrict__ U,
                                                     const double* __restrict__ ework, float* __restrict__ x_next) {
  __shared__ double es[32][kGB + 1];
  const int f0 = (g.block + 1) * kGB;
  const int r0 = blockIdx.y * 32;
  for (int e = threadIdx.x; e < 32 * kGB; e += 256) {
    const int rr = e / kGB, q = e % kGB;
    es[rr][q] = r0 + rr < g.rows ? ework[(size_t)(r0 + rr) * kGB + (size_t)q] : 0.0;
  }
  __syncthreads();
  const int c = f0 + blockIdx.x * 256 + threadIdx.x;
  if (c >= g.Kp) return;
  double u[kGB];
#pragma unroll
  for (int q = 0; q < kGB; ++q) u[q] = U[(size_t)(g.block * kGB + q) * g.Kp + (size_t)c];
  const int nr = min(32, g.rows - r0);
  for (int rr = 0; rr < nr; ++rr) {
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < kGB; ++q) s = fma(es[rr][q], u[q], s);
    double* wp = Wq + (size_t)(r0 + rr) * g.Kp + (size_t)c;
    const double w = *wp - s;
    *wp = w;
    if (c < f0 + kGB) x_next[(size_t)(r0 + rr) * kGB + (size_t)(c - f0)] = (float)w;
  }
}

// x_next for the direct variant (no update): the next block column as fp32
__global__ __launch_bounds__(256) void k_gptq_next(GptqCol g, const double* __restrict__ Wq, float* __restrict__ x_next) {
  const int f0 = (g.block + 1) * kGB;
  const size_t n = (size_t)g.rows * kGB;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) {
    const int r = (int)(e / kGB), q = (int)(e % kGB);
    x_next[e] = (float)Wq[(size_t)r * g.Kp + (size_t)(f0 + q)];
  }
}
