// Offline side on gfx950: the rank-r factors of the smoothed weight by a
// randomized truncated SVD.
//
// The 16-bit branch of the layer is the rank-r part of W_hat = W diag(lambda)
// from its SVD (Nunchaku troubleshooting page on apatero.com, section "O que
// e Nunchaku e como acelera modelos Qwen"; Nunchaku Lite page on axbrief.com,
// section "The Mechanics of 4-Bit Efficiency and SVDQuant").  The pages leave
// the SVD's algorithm open; this is the randomized range finder with power
// iterations of Halko, Martinsson and Tropp ("Finding structure with
// randomness", SIAM Review 2011, algorithms 4.4 and 5.1) with l = r + 16
// sketch columns:
//   Omega [N][l] Rademacher signs from Philox4x32-10;
//   Q = orth(W_hat^T Omega);  q times: Z = orth(W_hat Q), Q = orth(W_hat^T Z);
//   B = W_hat Q;  B^T B = V diag(s^2) V^T;  L1 = Q V_r diag(sqrt s),
//   L2^T = B V_r diag(1 / sqrt s);
// orth() is shifted CholeskyQR2.  Every step runs in fp64.
//
// Kernels:
//   * rsvd_product: the skinny products W_hat Q, W_hat^T Z (through a
//     transposed copy of W, so both are "rows of A times a small matrix"), the
//     CholeskyQR applications Y L^-T and the factor products, on the fp64
//     matrix cores (v_mfma_f64_16x16x4f64), split along the contraction into
//     fp64 partial sums that the next kernel adds in a fixed order;
//   * rsvd_sum_gram: adds the partials and forms the l x l Gram matrix Y^T Y
//     of a block of rows on the matrix cores; rsvd_gram_reduce adds the
//     blocks' Gram matrices in order;
//   * rsvd_chol_inv (one workgroup): shifted Cholesky G + d I = L L^T and
//     L^-1 in LDS;
//   * rsvd_jacobi (one workgroup): cyclic parallel Jacobi on B^T B in LDS,
//     logging every rotation; rsvd_vbuild replays the log to form V;
//     rsvd_finish orders the eigenpairs and scales the factor columns.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace svdq {

typedef double v4d __attribute__((ext_vector_type(4)));
typedef double v2d __attribute__((ext_vector_type(2)));

namespace {

constexpr int RSVD_OVERSAMPLE = 16;
constexpr int RSVD_MAX_L = 144;           // rank <= 128
constexpr int RSVD_MAX_LP = 144;          // l rounded up to 16
constexpr int RSVD_MAX_SWEEPS = 40;
constexpr double RSVD_SHIFT = 1e-12;
constexpr int GRAM_ROWS = 32;             // rows of Y per LDS chunk of rsvd_sum_gram
constexpr int GRAM_TILES_PER_WAVE = 12;   // 45 tiles of 16 x 16 at LP = 144, 4 waves

__device__ __forceinline__ v4d mfma_f64(double a, double b, v4d c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// Workgroup barrier for kernels whose waves share only LDS: waits for this
// wave's LDS operations (lgkmcnt(0); vmcnt and expcnt left at their maxima)
// and not for its global loads and stores, which __syncthreads() would drain.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
}

// ------------------------------------------------------------------ transpose
// Wt[k][n] = W[n][k] (bf16 bit patterns), 64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void rsvd_transpose_kernel(int N, int K,
                                                             const uint16_t* __restrict__ W,
                                                             uint16_t* __restrict__ Wt) {
  __shared__ uint16_t tile[64][66];
  const int n0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  const int row = t >> 2, col = (t & 3) * 16;
  const v4u* src = reinterpret_cast<const v4u*>(W + (int64_t)(n0 + row) * K + k0 + col);
  const v4u a = src[0], b = src[1];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    tile[row][col + 2 * e] = a[e] & 0xFFFFu;
    tile[row][col + 2 * e + 1] = a[e] >> 16;
    tile[row][col + 8 + 2 * e] = b[e] & 0xFFFFu;
    tile[row][col + 8 + 2 * e + 1] = b[e] >> 16;
  }
  __syncthreads();
  v4u oa, ob;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    oa[e] = tile[col + 2 * e][row] | ((uint32_t)tile[col + 2 * e + 1][row] << 16);
    ob[e] = tile[col + 8 + 2 * e][row] | ((uint32_t)tile[col + 8 + 2 * e + 1][row] << 16);
  }
  v4u* dst = reinterpret_cast<v4u*>(Wt + (int64_t)(k0 + row) * N + n0 + col);
  dst[0] = oa;
  dst[1] = ob;
}

// ------------------------------------------------------------------ sketch
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of two 32 x 32 -> 64-bit products
// with the round keys bumped by the Weyl constants between rounds.
__device__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(M0, c[0]), lo0 = M0 * c[0];
    const uint32_t hi1 = __umulhi(M1, c[2]), lo1 = M1 * c[2];
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

// Omega[n][j] = -1 if bit (j mod 128) of Philox(counter (n, j / 128, 0, 0),
// key (seed lo, seed hi)) is set, else +1, for j < l; 0 for l <= j < LP.
__global__ __launch_bounds__(256) void rsvd_omega_kernel(int N, int l, int LP, uint32_t seed_lo,
                                                         uint32_t seed_hi,
                                                         double* __restrict__ Om) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)N * LP) return;
  const int n = (int)(e / LP), j = (int)(e % LP);
  double v = 0.0;
  if (j < l) {
    uint32_t c[4] = {(uint32_t)n, (uint32_t)(j >> 7), 0u, 0u};
    philox4x32_10(c, seed_lo, seed_hi);
    const int b = j & 127;
    v = ((c[b >> 5] >> (b & 31)) & 1u) ? -1.0 : 1.0;
  }
  Om[e] = v;
}

// ------------------------------------------------------------------ products
// out[m][j] = sum_c A_hat[m][c] X[c][j] for 16 RB rows m per wave and 16 CB
// columns j, c over the contraction chunks of this split (blockIdx.z).
//   AT 0: A bf16 [rows][lda], A_hat = fp32(A * scale[c])   (W_hat);
//   AT 1: A bf16, A_hat = fp32(A * scale[m])               (W_hat^T via Wt);
//   AT 2: A fp64 [rows][lda], A_hat = A.
// A chunk is 32 (bf16) or 16 (fp64) contraction indices; in MFMA step t the
// lanes of slot g = lane / 16 take contraction index c0 + (chunk / 4) g + t,
// so each lane loads its A values with one contiguous 16-byte (bf16) or two
// 16-byte (fp64) loads per 16-row block.  The next chunk's A values are
// loaded while the current chunk runs, and each step's X values one step
// ahead (clamped to the last chunk, so every iteration issues the same
// loads).  Output:
//   OUT 0: fp64 partial sums out[split * ostride + m * old + j];
//   OUT 1: bf16 (RNE through fp32) out[m * old + j];
//   OUT 2: bf16 (RNE through fp32) transposed out[j * old + m].
// Column blocks at or past nblk are skipped (wave-uniform).
template <int AT, int RB>
struct AChunk {
  double ad[AT == 2 ? RB : 1][4];
  v4u wr[AT == 2 ? 1 : RB];
  float csc[8];
};

template <int AT, int RB, int CB, int OUT>
__global__ __launch_bounds__(256) void rsvd_product_kernel(
    int rows, int nchunks, int cps, const void* __restrict__ Aptr, int64_t lda,
    const float* __restrict__ scale, const double* __restrict__ X, int64_t ldx, int nblk,
    void* __restrict__ out, int64_t old, int64_t ostride) {
  constexpr int KC = AT == 2 ? 16 : 32;
  constexpr int ST = KC / 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = (blockIdx.x * 4 + wave) * 16 * RB;
  if (m0 >= rows) return;
  const int cb0 = blockIdx.y * CB;
  const int split = blockIdx.z;
  const int ch0 = split * cps;
  const int ch1 = min(nchunks, ch0 + cps);
  const int r16 = lane & 15, g = lane >> 4;

  v4d acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = v4d{0.0, 0.0, 0.0, 0.0};

  float rsc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) rsc[rb] = AT == 1 ? scale[m0 + 16 * rb + r16] : 1.f;

  auto load_a = [&](int ch, AChunk<AT, RB>& a) {
    const int c0 = ch * KC;
    if constexpr (AT == 2) {
      const double* A = static_cast<const double*>(Aptr);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const double* p = A + (int64_t)(m0 + 16 * rb + r16) * lda + c0 + 4 * g;
        const v2d x0 = *reinterpret_cast<const v2d*>(p);
        const v2d x1 = *reinterpret_cast<const v2d*>(p + 2);
        a.ad[rb][0] = x0[0];
        a.ad[rb][1] = x0[1];
        a.ad[rb][2] = x1[0];
        a.ad[rb][3] = x1[1];
      }
    } else {
      const uint16_t* A = static_cast<const uint16_t*>(Aptr);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        a.wr[rb] =
            *reinterpret_cast<const v4u*>(A + (int64_t)(m0 + 16 * rb + r16) * lda + c0 + 8 * g);
      if constexpr (AT == 0) {
        const v4f s0 = *reinterpret_cast<const v4f*>(scale + c0 + 8 * g);
        const v4f s1 = *reinterpret_cast<const v4f*>(scale + c0 + 8 * g + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a.csc[e] = s0[e];
          a.csc[4 + e] = s1[e];
        }
      }
    }
  };
  // X values of contraction row `row` for this lane's columns
  auto load_x = [&](int row, double (&xb)[CB]) {
    const double* xr = X + (int64_t)row * ldx + 16 * cb0 + r16;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) xb[cb] = (cb0 + cb < nblk) ? xr[16 * cb] : 0.0;
  };
  double xb[2][CB];
  auto run_chunk = [&](const AChunk<AT, RB>& a, int ch) {
#pragma unroll
    for (int t = 0; t < ST; ++t) {
      const int nch = t + 1 < ST ? ch : min(ch + 1, ch1 - 1);
      load_x(nch * KC + ST * g + (t + 1 < ST ? t + 1 : 0), xb[(t + 1) & 1]);
      double av[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if constexpr (AT == 2) {
          av[rb] = a.ad[rb][t];
        } else {
          const uint32_t h = (t & 1) ? (a.wr[rb][t >> 1] >> 16) : (a.wr[rb][t >> 1] & 0xFFFFu);
          av[rb] = (double)(bf16_to_f32(h) * (AT == 0 ? a.csc[t] : rsc[rb]));
        }
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (cb0 + cb < nblk) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) acc[rb][cb] = mfma_f64(av[rb], xb[t & 1][cb], acc[rb][cb]);
        }
      }
    }
  };

  if (ch0 < ch1) {
    AChunk<AT, RB> a0, a1;
    load_a(ch0, a0);
    load_x(ch0 * KC + ST * g, xb[0]);
    for (int ch = ch0; ch < ch1; ch += 2) {
      load_a(min(ch + 1, ch1 - 1), a1);
      run_chunk(a0, ch);
      if (ch + 1 >= ch1) break;
      load_a(min(ch + 2, ch1 - 1), a0);
      run_chunk(a1, ch + 1);
    }
  }

  // D lane layout of v_mfma_f64_16x16x4f64 on gfx950: element v of lane
  // 16 g + r16 is row g + 4 v, column r16 (the inputs: lane 16 g + r16 holds
  // A[r16][g] and B[g][r16]).
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if (cb0 + cb >= nblk) continue;
    const int col = 16 * (cb0 + cb) + r16;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = m0 + 16 * rb + g;
      if constexpr (OUT == 0) {
        double* o = static_cast<double*>(out) + split * ostride + (int64_t)row * old + col;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[4 * v * old] = acc[rb][cb][v];
      } else if constexpr (OUT == 1) {
        uint16_t* o = static_cast<uint16_t*>(out) + (int64_t)row * old + col;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[4 * v * old] = (uint16_t)f32_to_bf16((float)acc[rb][cb][v]);
      } else {
        uint16_t* o = static_cast<uint16_t*>(out) + (int64_t)col * old + row;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[4 * v] = (uint16_t)f32_to_bf16((float)acc[rb][cb][v]);
      }
    }
  }
}

// ------------------------------------------------------------------ Gram
// Rows [r0, r1) of Y = sum_s P[s] (s in order), written to Y when Y is not
// null, and this block's Gram matrix Gp[block] = Y_rows^T Y_rows on the
// 16 x 16 tiles (ib <= jb) of the LP x LP result, tile q of wave w being
// number w + 4 q of the row-major upper-triangle tile order.
__global__ __launch_bounds__(256) void rsvd_sum_gram_kernel(const double* __restrict__ P, int S,
                                                            int64_t pstride, int T, int LP,
                                                            int rpb, double* __restrict__ Y,
                                                            double* __restrict__ Gp) {
  __shared__ __attribute__((aligned(16))) double tile[GRAM_ROWS][RSVD_MAX_LP + 2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int nblk = LP / 16;
  const int ntiles = nblk * (nblk + 1) / 2;
  const int r0 = blockIdx.x * rpb;
  const int r1 = min(T, r0 + rpb);

  int tib[GRAM_TILES_PER_WAVE], tjb[GRAM_TILES_PER_WAVE];
#pragma unroll
  for (int q = 0; q < GRAM_TILES_PER_WAVE; ++q) {
    int id = wave + 4 * q, ib = 0;
    while (ib < nblk && id >= nblk - ib) {
      id -= nblk - ib;
      ++ib;
    }
    tib[q] = ib;
    tjb[q] = ib + id;
  }
  v4d acc[GRAM_TILES_PER_WAVE];
#pragma unroll
  for (int q = 0; q < GRAM_TILES_PER_WAVE; ++q) acc[q] = v4d{0.0, 0.0, 0.0, 0.0};

  const int half = LP / 2;
  for (int c0 = r0; c0 < r1; c0 += GRAM_ROWS) {
    for (int e = threadIdx.x; e < GRAM_ROWS * half; e += 256) {
      const int row = e / half, col = 2 * (e % half);
      v2d v = v2d{0.0, 0.0};
      if (c0 + row < r1) {
        const int64_t off = (int64_t)(c0 + row) * LP + col;
        for (int s = 0; s < S; ++s) v += *reinterpret_cast<const v2d*>(P + s * pstride + off);
        if (Y != nullptr) *reinterpret_cast<v2d*>(Y + off) = v;
      }
      *reinterpret_cast<v2d*>(&tile[row][col]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < GRAM_TILES_PER_WAVE; ++q) {
      if (wave + 4 * q < ntiles) {
#pragma unroll
        for (int st = 0; st < GRAM_ROWS / 4; ++st) {
          const double av = tile[4 * st + g][16 * tib[q] + r16];
          const double bv = tile[4 * st + g][16 * tjb[q] + r16];
          acc[q] = mfma_f64(av, bv, acc[q]);
        }
      }
    }
    __syncthreads();
  }
  double* gp = Gp + (int64_t)blockIdx.x * LP * LP;
#pragma unroll
  for (int q = 0; q < GRAM_TILES_PER_WAVE; ++q) {
    if (wave + 4 * q < ntiles) {
#pragma unroll
      for (int v = 0; v < 4; ++v) gp[(16 * tib[q] + g + 4 * v) * LP + 16 * tjb[q] + r16] = acc[q][v];
    }
  }
}

// G[x][y] = G[y][x] = sum_b Gp[b][x][y] for x <= y: 64 entries per
// workgroup, its 4 waves summing every 4th block (b = w, w + 4, ...), then
// the four sums added in wave order.
__global__ __launch_bounds__(256) void rsvd_gram_reduce_kernel(const double* __restrict__ Gp, int NB,
                                                               int LP, double* __restrict__ G) {
  __shared__ double part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int n = LP * LP;
  double acc = 0.0;
  if (e < n) {
    for (int b = wave; b < NB; b += 4) acc += Gp[(int64_t)b * n + e];
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && e < n) {
    const int x = e / LP, y = e % LP;
    if (x <= y) {
      const double v = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
      G[x * LP + y] = v;
      G[y * LP + x] = v;
    }
  }
}

// ------------------------------------------------------------------ Cholesky
__device__ __forceinline__ int tri(int i, int j) { return i * (i + 1) / 2 + j; }  // j <= i

// Row and column of entry e of the packed lower triangle.
__device__ __forceinline__ void tri_rc(int e, int& i, int& j) {
  int r = (int)((__builtin_sqrtf(8.0f * (float)e + 1.0f) - 1.0f) * 0.5f);
  while (r * (r + 1) / 2 > e) --r;
  while ((r + 1) * (r + 2) / 2 <= e) ++r;
  i = r;
  j = e - r * (r + 1) / 2;
}

// Shifted Cholesky of the l x l Gram matrix, G + (1e-12 trace(G) / l) I =
// L L^T (right-looking, one column per step), then L^-1 in place (row k of
// L^-1 is final once the contributions of rows 0..k-1 are added; each step
// adds row k's contribution to the rows below).  Output XT[c][j] = L^-1[j][c]
// (c <= j < l), zero elsewhere in LP x LP: the right operand of Y <- Y L^-T.
// A zero matrix (trace 0) gives XT = I, so a zero Y stays zero.  One thread
// per entry of a step (1024 threads).
constexpr int CHOL_THREADS = 1024;

__global__ __launch_bounds__(CHOL_THREADS) void rsvd_chol_inv_kernel(const double* __restrict__ G, int l,
                                                             int LP, double* __restrict__ XT) {
  __shared__ double a[RSVD_MAX_L * (RSVD_MAX_L + 1) / 2];
  __shared__ double colk[RSVD_MAX_L];
  __shared__ double s_trace;
  const int tid = threadIdx.x;
  const int nt = l * (l + 1) / 2;
  for (int e = tid; e < nt; e += CHOL_THREADS) {
    int i, j;
    tri_rc(e, i, j);
    a[e] = G[i * LP + j];
  }
  if (tid == 0) {
    double tr = 0.0;
    for (int i = 0; i < l; ++i) tr += G[i * LP + i];
    s_trace = tr;
  }
  lds_barrier();
  const double tr = s_trace;
  if (tr == 0.0) {
    for (int e = tid; e < LP * LP; e += CHOL_THREADS) {
      const int c = e / LP, j = e % LP;
      XT[e] = (c == j && j < l) ? 1.0 : 0.0;
    }
    return;
  }
  const double shift = RSVD_SHIFT * tr / (double)l;
  for (int i = tid; i < l; i += CHOL_THREADS) a[tri(i, i)] += shift;
  lds_barrier();

  for (int j = 0; j < l; ++j) {
    const double d = __builtin_sqrt(a[tri(j, j)]);
    for (int i = j + 1 + tid; i < l; i += CHOL_THREADS) a[tri(i, j)] /= d;
    lds_barrier();
    const int m = l - j - 1;
    const int cnt = m * (m + 1) / 2;
    for (int e = tid; e < cnt; e += CHOL_THREADS) {
      int ii, kk;
      tri_rc(e, ii, kk);
      ii += j + 1;
      kk += j + 1;
      a[tri(ii, kk)] -= a[tri(ii, j)] * a[tri(kk, j)];
    }
    if (tid == 0) a[tri(j, j)] = d;
    lds_barrier();
  }

  for (int k = 0; k < l; ++k) {
    const double dk = a[tri(k, k)];
    for (int e = tid; e < l; e += CHOL_THREADS) {
      if (e < k) a[tri(k, e)] = -a[tri(k, e)] / dk;
      else if (e > k) colk[e] = a[tri(e, k)];
    }
    lds_barrier();
    const double inv = 1.0 / dk;
    if (tid == 0) a[tri(k, k)] = inv;
    const int rows_below = l - k - 1;
    const int cnt = rows_below * (k + 1);
    for (int e = tid; e < cnt; e += CHOL_THREADS) {
      const int i = k + 1 + e / (k + 1), j = e % (k + 1);
      const double xk = j < k ? a[tri(k, j)] : inv;
      const double prev = j < k ? a[tri(i, j)] : 0.0;
      a[tri(i, j)] = prev + colk[i] * xk;
    }
    lds_barrier();
  }

  for (int e = tid; e < LP * LP; e += CHOL_THREADS) {
    const int c = e / LP, j = e % LP;
    XT[e] = (c <= j && j < l) ? a[tri(j, c)] : 0.0;
  }
}

// ------------------------------------------------------------------ Jacobi
// Index at position p of step k of the round-robin ordering of le (even)
// indices: position 0 stays, the others rotate.
__device__ __forceinline__ int rr_index(int p, int k, int le) {
  int v = p - 1 + k;            // 0 <= p - 1 + k < 2 (le - 1): one conditional subtraction
  v = v >= le - 1 ? v - (le - 1) : v;
  return p == 0 ? 0 : 1 + v;
}

__device__ __forceinline__ int sym(int x, int y) { return x >= y ? tri(x, y) : tri(y, x); }

// Cyclic Jacobi on the symmetric l x l matrix C (Golub and Van Loan, "Matrix
// Computations", the symmetric Schur decomposition by plane rotations
// J(p, q) with J_pp = J_qq = c, J_pq = s, J_qp = -s, C <- J^T C J), in the
// round-robin parallel order: each step rotates le / 2 disjoint pairs at once,
// every 2 x 2 block of C (rows of one pair, columns of another) being
// rotated by one thread.  A pair rotates when |c_pq| > 2^-52 sqrt|c_pp c_qq|;
// the sweeps stop after one with no rotation (at most 40).  Every step's
// (c, s) per pair goes to the log rot[sweep][step][pair]; ev[i] is the final
// diagonal, nsweeps the number of sweeps logged.  One thread per pair block
// (1024 threads, at most 3 blocks each).
constexpr int JAC_THREADS = 1024;

__global__ __launch_bounds__(JAC_THREADS) void rsvd_jacobi_kernel(const double* __restrict__ Cm, int l,
                                                           int LP, double* __restrict__ rot,
                                                           double* __restrict__ ev,
                                                           int* __restrict__ nsweeps) {
  __shared__ double a[RSVD_MAX_L * (RSVD_MAX_L + 1) / 2];
  __shared__ double pc[RSVD_MAX_L / 2], ps[RSVD_MAX_L / 2], pt[RSVD_MAX_L / 2];
  __shared__ int pp[RSVD_MAX_L / 2], pq[RSVD_MAX_L / 2];
  __shared__ int s_count;
  const int tid = threadIdx.x;
  const int nt = l * (l + 1) / 2;
  for (int e = tid; e < nt; e += JAC_THREADS) {
    int i, j;
    tri_rc(e, i, j);
    a[e] = Cm[i * LP + j];
  }
  const int le = l + (l & 1), h = le / 2, nsteps = le - 1;
  // this thread's pair blocks (a <= b), at most 3 (h <= 72: 2628 blocks)
  const int nblocks = h * (h + 1) / 2;
  int ba[3], bb[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    int id = tid + JAC_THREADS * q, x = 0;
    if (id < nblocks) {
      while (id >= h - x) {
        id -= h - x;
        ++x;
      }
      ba[q] = x;
      bb[q] = x + id;
    } else {
      ba[q] = bb[q] = -1;
    }
  }
  constexpr double EPS = 2.220446049250313e-16;
  int sweep = 0;
  while (sweep < RSVD_MAX_SWEEPS) {
    if (tid == 0) s_count = 0;
    lds_barrier();
    for (int k = 0; k < nsteps; ++k) {
      if (tid < h) {
        const int u = rr_index(tid, k, le), w = rr_index(le - 1 - tid, k, le);
        const int p = min(u, w), q = max(u, w);
        double c = 1.0, s = 0.0, t = 0.0;
        if (q < l) {
          const double app = a[tri(p, p)], aqq = a[tri(q, q)], apq = a[tri(q, p)];
          if (apq != 0.0 && fabs(apq) > EPS * __builtin_sqrt(fabs(app) * fabs(aqq))) {
            const double tau = (aqq - app) / (2.0 * apq);
            const double at = fabs(tau);
            const double den = at > 1.0 ? at * (1.0 + __builtin_sqrt(1.0 + (1.0 / at) / at))
                                        : at + __builtin_sqrt(1.0 + at * at);
            t = (tau >= 0.0 ? 1.0 : -1.0) / den;
            c = 1.0 / __builtin_sqrt(1.0 + t * t);
            s = t * c;
            atomicAdd(&s_count, 1);
          }
        }
        pc[tid] = c;
        ps[tid] = s;
        pt[tid] = t;
        pp[tid] = p;
        pq[tid] = q;
        double* lg = rot + ((int64_t)(sweep * nsteps + k) * h + tid) * 2;
        lg[0] = c;
        lg[1] = s;
      }
      lds_barrier();
#pragma unroll
      for (int q3 = 0; q3 < 3; ++q3) {
        const int x = ba[q3], y = bb[q3];
        if (x < 0) continue;
        if (x == y) {
          const int p = pp[x], q = pq[x];
          if (pt[x] != 0.0) {
            const double apq = a[tri(q, p)];
            a[tri(p, p)] -= pt[x] * apq;
            a[tri(q, q)] += pt[x] * apq;
            a[tri(q, p)] = 0.0;
          }
          continue;
        }
        const double ca = pc[x], sa = ps[x], cb = pc[y], sb = ps[y];
        if (sa == 0.0 && sb == 0.0) continue;
        const int pa = pp[x], qa = pq[x], pb = pp[y], qb = pq[y];
        const bool va = qa < l, vb = qb < l;  // the dummy index (odd l) has no entries
        const double e00 = a[sym(pa, pb)];
        const double e01 = vb ? a[sym(pa, qb)] : 0.0;
        const double e10 = va ? a[sym(qa, pb)] : 0.0;
        const double e11 = (va && vb) ? a[sym(qa, qb)] : 0.0;
        const double r00 = ca * e00 - sa * e10, r01 = ca * e01 - sa * e11;
        const double r10 = sa * e00 + ca * e10, r11 = sa * e01 + ca * e11;
        a[sym(pa, pb)] = cb * r00 - sb * r01;
        if (vb) a[sym(pa, qb)] = sb * r00 + cb * r01;
        if (va) a[sym(qa, pb)] = cb * r10 - sb * r11;
        if (va && vb) a[sym(qa, qb)] = sb * r10 + cb * r11;
      }
      lds_barrier();
    }
    ++sweep;
    const int cnt = s_count;
    lds_barrier();
    if (cnt == 0) break;
  }
  for (int i = tid; i < l; i += JAC_THREADS) ev[i] = a[tri(i, i)];
  if (tid == 0) *nsweeps = sweep;
}

// V = J_1 J_2 ... (the logged rotations in order): rows 16 blockIdx.x ..
// +15 of V, each row vector rotated in LDS.  V[i][c] is component i of
// eigenvector c.  Columns l..LP-1 are zero.
constexpr int VB_THREADS = 1024;
constexpr int VB_ITEMS = 2;   // ceil(16 * 72 / 1024)

__global__ __launch_bounds__(VB_THREADS) void rsvd_vbuild_kernel(const double* __restrict__ rot,
                                                                 const int* __restrict__ nsweeps,
                                                                 int l, int LP,
                                                                 double* __restrict__ V) {
  __shared__ double vr[16][RSVD_MAX_LP];
  const int i0 = blockIdx.x * 16;
  for (int e = threadIdx.x; e < 16 * LP; e += VB_THREADS) {
    const int rho = e / LP, c = e % LP;
    vr[rho][c] = (i0 + rho == c) ? 1.0 : 0.0;
  }
  const int le = l + (l & 1), h = le / 2, nsteps = le - 1;
  const int total = *nsweeps * nsteps;   // logged steps, in order
  // this thread's (row, pair) items are fixed; each step's (c, s) are loaded
  // one step ahead
  int rho[VB_ITEMS], xi[VB_ITEMS];
#pragma unroll
  for (int z = 0; z < VB_ITEMS; ++z) {
    const int e = threadIdx.x + z * VB_THREADS;
    rho[z] = e < 16 * h ? e / h : -1;
    xi[z] = e % h;
  }
  double cn[VB_ITEMS], sn[VB_ITEMS];
#pragma unroll
  for (int z = 0; z < VB_ITEMS; ++z) {
    cn[z] = total > 0 && rho[z] >= 0 ? rot[2 * xi[z]] : 1.0;
    sn[z] = total > 0 && rho[z] >= 0 ? rot[2 * xi[z] + 1] : 0.0;
  }
  for (int st = 0; st < total; ++st) {
    const int k = st % nsteps;
    const int nxt = min(st + 1, total - 1);
    double c[VB_ITEMS], s[VB_ITEMS];
#pragma unroll
    for (int z = 0; z < VB_ITEMS; ++z) {
      c[z] = cn[z];
      s[z] = sn[z];
      if (rho[z] >= 0) {
        const double* lg = rot + ((int64_t)nxt * h + xi[z]) * 2;
        cn[z] = lg[0];
        sn[z] = lg[1];
      }
    }
    lds_barrier();
    double vp[VB_ITEMS], vq[VB_ITEMS];
    int p[VB_ITEMS], q[VB_ITEMS];
#pragma unroll
    for (int z = 0; z < VB_ITEMS; ++z) {
      const int u = rr_index(xi[z], k, le), w = rr_index(le - 1 - xi[z], k, le);
      p[z] = min(u, w);
      q[z] = max(u, w);
      if (rho[z] >= 0 && s[z] != 0.0 && q[z] < l) {
        vp[z] = vr[rho[z]][p[z]];
        vq[z] = vr[rho[z]][q[z]];
      }
    }
#pragma unroll
    for (int z = 0; z < VB_ITEMS; ++z) {
      if (rho[z] < 0 || s[z] == 0.0 || q[z] >= l) continue;
      vr[rho[z]][p[z]] = c[z] * vp[z] - s[z] * vq[z];
      vr[rho[z]][q[z]] = s[z] * vp[z] + c[z] * vq[z];
    }
  }
  lds_barrier();
  for (int e = threadIdx.x; e < 16 * LP; e += VB_THREADS) {
    const int r = e / LP, c = e % LP;
    if (i0 + r < l) V[(int64_t)(i0 + r) * LP + c] = c < l ? vr[r][c] : 0.0;
  }
}

// Orders the eigenpairs by descending eigenvalue (equal ones by index), fixes
// each eigenvector's sign so that its largest-magnitude component (the first
// if several) is positive, and writes for output column o < r with
// eigenpair (e, v):  s_o = sqrt(max(e, 0)),  F1[c][o] = v_c sqrt(s_o),
// F2[c][o] = v_c / sqrt(s_o) (v_c when s_o = 0), rows l..LP-1 zero;
// sigma[o] = s_o when sigma is not null.
__global__ __launch_bounds__(256) void rsvd_finish_kernel(const double* __restrict__ ev,
                                                          const double* __restrict__ V, int l,
                                                          int LP, int r, double* __restrict__ F1,
                                                          double* __restrict__ F2,
                                                          double* __restrict__ sigma) {
  for (int e = threadIdx.x; e < (LP - l) * r; e += 256) {
    F1[(int64_t)l * r + e] = 0.0;
    F2[(int64_t)l * r + e] = 0.0;
  }
  for (int i = threadIdx.x; i < l; i += 256) {
    const double ei = ev[i];
    int pos = 0;
    for (int j = 0; j < l; ++j) {
      const double ej = ev[j];
      pos += (ej > ei || (ej == ei && j < i)) ? 1 : 0;
    }
    if (pos >= r) continue;
    int big = 0;
    double bmax = -1.0;
    for (int c = 0; c < l; ++c) {
      const double m = fabs(V[(int64_t)c * LP + i]);
      if (m > bmax) {
        bmax = m;
        big = c;
      }
    }
    const double sgn = V[(int64_t)big * LP + i] < 0.0 ? -1.0 : 1.0;
    const double so = __builtin_sqrt(fmax(ei, 0.0));
    const double rs = __builtin_sqrt(so);
    const double rdiv = rs > 0.0 ? rs : 1.0;
    for (int c = 0; c < l; ++c) {
      const double vc = sgn * V[(int64_t)c * LP + i];
      F1[(int64_t)c * r + pos] = vc * rs;
      F2[(int64_t)c * r + pos] = vc / rdiv;
    }
    if (sigma != nullptr) sigma[pos] = so;
  }
}

// ------------------------------------------------------------------ host plan
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Split {
  int S, cps, nchunks;
};

// Split of a product's contraction (nchunks chunks) so that the grid has
// about 2048 waves, each split at least 4 chunks, no split empty.
Split plan_split(int rows, int nchunks, int cg) {
  const int waves = (rows / 64) * cg;
  int S = (2048 + waves - 1) / waves;
  S = std::max(1, std::min(S, std::max(1, nchunks / 4)));
  const int cps = (nchunks + S - 1) / S;
  S = (nchunks + cps - 1) / cps;
  return Split{S, cps, nchunks};
}

int col_groups(int nblk) { return (nblk + 3) / 4; }
int col_blocks(int nblk) {
  const int cg = col_groups(nblk);
  return (nblk + cg - 1) / cg;
}

struct GramPlan {
  int NB, rpb;
};
GramPlan plan_gram(int T) {
  const int chunks = (T + GRAM_ROWS - 1) / GRAM_ROWS;
  const int rpb = GRAM_ROWS * ((chunks + 511) / 512);
  return GramPlan{(T + rpb - 1) / rpb, rpb};
}

struct RsvdPlan {
  int N, K, r, l, LP, le;
  Split left, right;  // contraction K (rows N), contraction N (rows K)
  GramPlan gN, gK;
  size_t wt, z, q, y, t, p, gp, g, xt, rot, ev, ns, v, f1, f2, total;
};

RsvdPlan make_plan(int N, int K, int r) {
  RsvdPlan P{};
  P.N = N;
  P.K = K;
  P.r = r;
  P.l = std::min(r + RSVD_OVERSAMPLE, std::min(N, K));
  P.LP = (P.l + 15) / 16 * 16;
  P.le = P.l + (P.l & 1);
  const int cg = col_groups(P.LP / 16);
  P.left = plan_split(N, K / 32, cg);
  P.right = plan_split(K, N / 32, cg);
  P.gN = plan_gram(N);
  P.gK = plan_gram(K);
  const size_t LP = P.LP, rows = (size_t)std::max(N, K);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  P.wt = take((size_t)N * K * 2);
  P.z = take((size_t)N * LP * 8);
  P.q = take((size_t)K * LP * 8);
  P.y = take(rows * LP * 8);
  P.t = take(rows * LP * 8);
  P.p = take((size_t)std::max((size_t)P.left.S * N, (size_t)P.right.S * K) * LP * 8);
  P.gp = take((size_t)std::max(P.gN.NB, P.gK.NB) * LP * LP * 8);
  P.g = take(LP * LP * 8);
  P.xt = take(LP * LP * 8);
  P.rot = take((size_t)RSVD_MAX_SWEEPS * (P.le - 1) * (P.le / 2) * 2 * 8);
  P.ev = take(LP * 8);
  P.ns = take(16);
  P.v = take(LP * LP * 8);
  P.f1 = take(LP * r * 8);
  P.f2 = take(LP * r * 8);
  P.total = off;
  return P;
}

template <int AT, int OUT, int RB, int CB>
hipError_t product_cb(int rows, const Split& sp, const void* A, int64_t lda, const float* scale,
                      const double* X, int64_t ldx, int nblk, void* out, int64_t old,
                      int64_t ostride, hipStream_t s) {
  const dim3 grid((rows + 64 * RB - 1) / (64 * RB), (nblk + CB - 1) / CB, sp.S);
  hipLaunchKernelGGL((rsvd_product_kernel<AT, RB, CB, OUT>), grid, dim3(256), 0, s, rows,
                     sp.nchunks, sp.cps, A, lda, scale, X, ldx, nblk, out, old, ostride);
  return hipGetLastError();
}

// The W_hat products (bf16 A) use 64 rows per wave; the small fp64 products
// (CholeskyQR applications, factors) 16 rows per wave, for more waves.
template <int AT, int OUT>
hipError_t product(int rows, const Split& sp, const void* A, int64_t lda, const float* scale,
                   const double* X, int64_t ldx, int nblk, void* out, int64_t old,
                   int64_t ostride, hipStream_t s) {
  constexpr int RB = AT == 2 ? 1 : 4;
  switch (col_blocks(nblk)) {
    case 1: return product_cb<AT, OUT, RB, 1>(rows, sp, A, lda, scale, X, ldx, nblk, out, old, ostride, s);
    case 2: return product_cb<AT, OUT, RB, 2>(rows, sp, A, lda, scale, X, ldx, nblk, out, old, ostride, s);
    case 3: return product_cb<AT, OUT, RB, 3>(rows, sp, A, lda, scale, X, ldx, nblk, out, old, ostride, s);
    default: return product_cb<AT, OUT, RB, 4>(rows, sp, A, lda, scale, X, ldx, nblk, out, old, ostride, s);
  }
}

#define RSVD_TRY(expr)                       \
  do {                                       \
    const hipError_t e_ = (expr);            \
    if (e_ != hipSuccess) return e_;         \
  } while (0)

struct Ws {
  const RsvdPlan& P;
  uint8_t* base;
  double* d(size_t off) const { return reinterpret_cast<double*>(base + off); }
};

// Gram of the rows of sum_s Psum[s] ([T][LP]); writes that sum to Y when
// Y is not null; G (LP x LP) in the workspace.
hipError_t gram(const Ws& w, const double* Psum, int S, int64_t pstride, int T, const GramPlan& gp,
                double* Y, hipStream_t s) {
  const int LP = w.P.LP;
  hipLaunchKernelGGL(rsvd_sum_gram_kernel, dim3(gp.NB), dim3(256), 0, s, Psum, S, pstride, T, LP,
                     gp.rpb, Y, w.d(w.P.gp));
  RSVD_TRY(hipGetLastError());
  hipLaunchKernelGGL(rsvd_gram_reduce_kernel, dim3((LP * LP + 63) / 64), dim3(256), 0, s,
                     w.d(w.P.gp), gp.NB, LP, w.d(w.P.g));
  return hipGetLastError();
}

// dst = orth(sum_s Psum[s]) by shifted CholeskyQR2; T rows.
hipError_t orth(const Ws& w, const double* Psum, int S, int64_t pstride, int T,
                const GramPlan& gp, double* dst, hipStream_t s) {
  const RsvdPlan& P = w.P;
  const int LP = P.LP, nblk = LP / 16;
  const Split one{1, LP / 16, LP / 16};
  const double* Y = Psum;
  if (S > 1) Y = w.d(P.y);
  RSVD_TRY(gram(w, Psum, S, pstride, T, gp, S > 1 ? w.d(P.y) : nullptr, s));
  hipLaunchKernelGGL(rsvd_chol_inv_kernel, dim3(1), dim3(CHOL_THREADS), 0, s, w.d(P.g), P.l, LP, w.d(P.xt));
  RSVD_TRY(hipGetLastError());
  RSVD_TRY((product<2, 0>(T, one, Y, LP, nullptr, w.d(P.xt), LP, nblk, w.d(P.t), LP, 0, s)));
  RSVD_TRY(gram(w, w.d(P.t), 1, 0, T, gp, nullptr, s));
  hipLaunchKernelGGL(rsvd_chol_inv_kernel, dim3(1), dim3(CHOL_THREADS), 0, s, w.d(P.g), P.l, LP, w.d(P.xt));
  RSVD_TRY(hipGetLastError());
  return product<2, 0>(T, one, w.d(P.t), LP, nullptr, w.d(P.xt), LP, nblk, dst, LP, 0, s);
}

}  // namespace

size_t lowrank_factors_workspace_bytes(int N, int K, int rank) {
  return make_plan(N, K, rank).total;
}

// The workspace of the entry point that allocates nothing: a device array of
// fixed size in this library's code object, one copy per device, held until
// the process ends.  Host code never uses the array's name as an address;
// it asks the runtime for each device's copy once (with that device
// current) and passes that pointer to the kernels like a caller's workspace.
static __device__ __align__(256) uint8_t scratch[LOWRANK_STATIC_WORKSPACE];

hipError_t lowrank_static_workspace(void** ptr) {
  static std::mutex mu;
  static void* per_device[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_lowrank_factors(int N, int K, int rank, const uint16_t* W, const float* lambda,
                                  uint64_t seed, int power_iters, uint16_t* lora_down,
                                  uint16_t* lora_up, double* sigma, void* workspace,
                                  hipStream_t s) {
  const RsvdPlan P = make_plan(N, K, rank);
  const Ws w{P, static_cast<uint8_t*>(workspace)};
  const int LP = P.LP, nblk = LP / 16;
  uint16_t* Wt = reinterpret_cast<uint16_t*>(w.base + P.wt);
  double* Z = w.d(P.z);
  double* Q = w.d(P.q);
  double* Pp = w.d(P.p);

  hipLaunchKernelGGL(rsvd_transpose_kernel, dim3(K / 64, N / 64), dim3(256), 0, s, N, K, W, Wt);
  RSVD_TRY(hipGetLastError());
  const int64_t nz = (int64_t)N * LP;
  hipLaunchKernelGGL(rsvd_omega_kernel, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, s, N,
                     P.l, LP, (uint32_t)seed, (uint32_t)(seed >> 32), Z);
  RSVD_TRY(hipGetLastError());

  const int64_t strideK = (int64_t)K * LP, strideN = (int64_t)N * LP;
  // Q = orth(W_hat^T Omega)
  RSVD_TRY((product<1, 0>(K, P.right, Wt, N, lambda, Z, LP, nblk, Pp, LP, strideK, s)));
  RSVD_TRY(orth(w, Pp, P.right.S, strideK, K, P.gK, Q, s));
  for (int it = 0; it < power_iters; ++it) {
    RSVD_TRY((product<0, 0>(N, P.left, W, K, lambda, Q, LP, nblk, Pp, LP, strideN, s)));
    RSVD_TRY(orth(w, Pp, P.left.S, strideN, N, P.gN, Z, s));
    RSVD_TRY((product<1, 0>(K, P.right, Wt, N, lambda, Z, LP, nblk, Pp, LP, strideK, s)));
    RSVD_TRY(orth(w, Pp, P.right.S, strideK, K, P.gK, Q, s));
  }
  // B = W_hat Q, C = B^T B, eigenpairs of C
  RSVD_TRY((product<0, 0>(N, P.left, W, K, lambda, Q, LP, nblk, Pp, LP, strideN, s)));
  double* B = P.left.S > 1 ? Z : Pp;
  RSVD_TRY(gram(w, Pp, P.left.S, strideN, N, P.gN, P.left.S > 1 ? Z : nullptr, s));
  hipLaunchKernelGGL(rsvd_jacobi_kernel, dim3(1), dim3(JAC_THREADS), 0, s, w.d(P.g), P.l, LP,
                     w.d(P.rot), w.d(P.ev), reinterpret_cast<int*>(w.base + P.ns));
  RSVD_TRY(hipGetLastError());
  hipLaunchKernelGGL(rsvd_vbuild_kernel, dim3((P.l + 15) / 16), dim3(VB_THREADS), 0, s, w.d(P.rot),
                     reinterpret_cast<const int*>(w.base + P.ns), P.l, LP, w.d(P.v));
  RSVD_TRY(hipGetLastError());
  hipLaunchKernelGGL(rsvd_finish_kernel, dim3(1), dim3(256), 0, s, w.d(P.ev), w.d(P.v), P.l, LP,
                     rank, w.d(P.f1), w.d(P.f2), sigma);
  RSVD_TRY(hipGetLastError());
  // lora_down = (Q F1)^T [r][K], lora_up = B F2 [N][r]
  const Split one{1, LP / 16, LP / 16};
  RSVD_TRY((product<2, 2>(K, one, Q, LP, nullptr, w.d(P.f1), rank, rank / 16, lora_down, K, 0, s)));
  return product<2, 1>(N, one, B, LP, nullptr, w.d(P.f2), rank, rank / 16, lora_up, rank, 0, s);
}

}  // namespace svdq
