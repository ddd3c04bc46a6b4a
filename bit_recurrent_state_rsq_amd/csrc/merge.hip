// Low-Rank Bypass merge ("Preserving Updates in Low-Bit Recurrent State
// Quantization": abstract and Fig. 3 — small updates collect in a low-rank
// buffer and its sufficiently large elements are written into the quantized
// state every m steps; Table 6 gives k, m and the threshold eps_L).
//
// Per tile, with n bypass columns U (d_k x n) and W (d_v x n) in binary16:
//   L = U W^T                 column by column in index order; every fp16
//                             product is exact in float32, so each step is
//                             one FMA and L is the same float32 value the
//                             sequential sum gives
//   M = |L| > fl(eps_L s)     the elements that are large enough to store
//   x = M ? fl(s_hat + L) : s_hat,  s_hat = fl(c s)
//   step sizes from x (dynamic / persistent), codes RNE(x RN(1/s')), clamped;
//   BDR toward sign(L) on M with the no-update value s_hat as reference
//   R = L on not-M           the rest stays in the bypass as its best rank-k
//                             approximation (Eckart-Young), stored as balanced
//                             binary16 factors U_k S^1/2, V_k S^1/2 with the
//                             largest-magnitude stored entry of every U column
//                             positive (the first one on ties)
//
// The rank-k approximation is a subspace iteration started from the bypass's
// own right factors W (the row space of L), a fixed number of rounds of
//   Q <- orth(R Z);  Z <- R^T Q
// with CholeskyQR2 as orth, then Rayleigh-Ritz: the p x p matrix Z^T Z is
// diagonalised by cyclic Jacobi and its top k eigenpairs give the factors.
// R stays in registers in the decode kernel's 8x8-chunk lane layout; the
// bases, partial sums and the small matrices live in LDS.
#include <algorithm>

#include "rsq_kernels.hpp"
#include "lane_ops.hpp"

namespace rsq {

// Subspace iterations: each one shrinks the error of the rank-k subspace by
// about (sigma_(p+1) / sigma_k)^2, so a narrow bypass (few columns per kept
// rank) needs more of them. With the warm start these bring the Frobenius
// error within 1e-4 of the Eckart-Young optimum on the workloads' residuals.
constexpr int kMergeItersWide = 5;    // p >= 4k + 4
constexpr int kMergeItersNarrow = 12;
constexpr int kJacobiSweeps = 12;  // upper bound; stops once the off-diagonal part is negligible
constexpr int kChunkMin = 8, kChunkMax = 32;   // basis columns per cross-wavefront reduction pass
constexpr int kSm = kMaxCap + 1;   // row stride of the small p x p matrices
// misc block layout (floats)
constexpr int kMiscDinv = 0, kMiscOrder = kMaxCap, kMiscSroot = 2 * kMaxCap, kMiscFlag = 3 * kMaxCap,
              kMiscSign = 4 * kMaxCap, kMiscRot = 5 * kMaxCap, kMiscFloats = 7 * kMaxCap;

// LDS carve-up of the merge kernel (floats); the host sizes the launch with
// merge_lds_floats().
struct MergeLds {
  float* zt;    // [cap][zs]       right basis, column c at zt + c * zs
  float* yt;    // [cap][ys]       left basis
  float* part;  // [stripes][chunk][rows]  per-wavefront-stripe partial sums
  float* g;     // [kMaxCap][kSm]  Gram matrix / Cholesky factor
  float* h0;    // [kMaxCap][kSm]  Jacobi: H, double buffered
  float* h1;
  float* v0;    // [kMaxCap][kSm]  Jacobi: eigenvectors, double buffered
  float* v1;
  float* misc;  // [kMiscFloats]   1/diag of the Cholesky factor, eigen order, sigma^1/2,
                //                 the Jacobi stop flag, column signs
};

__host__ __device__ inline int merge_zs(int dv) { return dv + 4; }
__host__ __device__ inline int merge_ys(int dk) { return dk + 4; }

constexpr int kTri = kMaxCap * (kMaxCap + 1) / 2;   // entries of a symmetric kMaxCap x kMaxCap matrix

// floats of the partial-sum area: product stripes, or per-wavefront Gram partials
__host__ __device__ inline size_t merge_part_floats(int dk, int dv, int wrw, int wcw, int chunk) {
  const size_t prod = (size_t)chunk * (size_t)(wcw * dk > wrw * dv ? wcw * dk : wrw * dv);
  const size_t gram = (size_t)wrw * wcw * kTri;
  return prod > gram ? prod : gram;
}

size_t merge_lds_floats(int dk, int dv, int wrw, int wcw, int cap, int chunk) {
  const size_t part = merge_part_floats(dk, dv, wrw, wcw, chunk);
  return (size_t)cap * merge_zs(dv) + (size_t)cap * merge_ys(dk) + part + 5 * kMaxCap * kSm + kMiscFloats;
}

// sum over the CL column lanes of a wavefront (lane bits 0 .. log2(CL)-1);
// every lane of the group ends with the same value (the adds commute)
template <int CL>
__device__ __forceinline__ float col_lane_sum(float v) {
  v = __fadd_rn(v, dpp_xor1(v));
  v = __fadd_rn(v, dpp_xor2(v));
  if constexpr (CL >= 8)
    v = __fadd_rn(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  if constexpr (CL >= 16)
    v = __fadd_rn(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

__device__ __forceinline__ bool any_lane(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void load_half8(const __half* p, float out[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    out[2 * q] = __half2float(__ushort_as_half((uint16_t)(w[q] & 0xFFFFu)));
    out[2 * q + 1] = __half2float(__ushort_as_half((uint16_t)(w[q] >> 16)));
  }
}

// (a, b) with a <= b of the pi-th entry of the upper triangle of a p x p matrix, row by row
__device__ __forceinline__ void tri_pair(int pi, int p, int& a, int& b) {
  a = 0;
  int rowlen = p;
  while (pi >= rowlen) {
    pi -= rowlen;
    ++a;
    --rowlen;
  }
  b = a + pi;
}

template <int CL>
struct Merge {
  static constexpr int RL = 64 / CL;
  static constexpr int NB = (RL == 16) ? 4 : (RL == 8) ? 3 : 2;
  static constexpr int WR = 8 * RL;
  static constexpr int WC = 8 * CL;
  static constexpr int NSLOT = 8 >> (NB < 3 ? NB : 3);

  struct Geo {
    int wave, lane, nw, wrw, wcw, wr, wc, lc, i0, j0;
  };

  static __device__ __forceinline__ Geo geo(const StepArgs& a) {
    Geo g;
    g.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    g.lane = threadIdx.x & 63;
    g.nw = blockDim.x >> 6;
    g.wrw = a.dk / WR;
    g.wcw = a.dv / WC;
    g.wr = g.wave % g.wrw;
    g.wc = g.wave / g.wrw;
    g.lc = g.lane % CL;
    const int lr = g.lane / CL;
    const int rho = (int)(__builtin_bitreverse32((uint32_t)lr) >> (32 - NB));
    g.i0 = g.wr * WR + 8 * rho;
    g.j0 = g.wc * WC + 8 * g.lc;
    return g;
  }

  // ------------------------------------------------------------ merge into the codes
  // U and W (binary16) of the tile into LDS, column-major like in memory
  static __device__ __forceinline__ void stage_bypass(const StepArgs& a, const HeadEntry& he, const uint8_t* tb,
                                                      __half* us, __half* ws) {
    const uint4* U = reinterpret_cast<const uint4*>(tb + he.bypass_u);
    const uint4* W = reinterpret_cast<const uint4*>(tb + he.bypass_w);
    const int nu = a.n * a.dk / 8, nwv = a.n * a.dv / 8;   // 16-byte pieces
    for (int e = threadIdx.x; e < nu; e += blockDim.x) reinterpret_cast<uint4*>(us)[e] = U[e];
    for (int e = threadIdx.x; e < nwv; e += blockDim.x) reinterpret_cast<uint4*>(ws)[e] = W[e];
    __syncthreads();
  }

  // L = U W^T for the lane's chunk, in column index order (one FMA per column:
  // each binary16 product is exact in float32)
  static __device__ __forceinline__ void low_rank(const StepArgs& a, const Geo& g, const __half* us,
                                                  const __half* ws, float L[8][8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) L[i][j] = 0.f;
    for (int c = 0; c < a.n; ++c) {
      float u8[8], w8[8];
      load_half8(us + (size_t)c * a.dk + g.i0, u8);
      load_half8(ws + (size_t)c * a.dv + g.j0, w8);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) L[i][j] = __builtin_fmaf(u8[i], w8[j], L[i][j]);
    }
  }

  // Moves the elements of L above the threshold into the codes and
  // requantizes the chunk. Leaves in mk[i] the moved elements of row i:
  // bit j when L_ij > 0, bit 8+j when L_ij < 0.
  template <int BITS>
  static __device__ __forceinline__ void requantize(const StepArgs& a, const HeadEntry& he, uint8_t* tb, const Geo& g,
                                                    const __half* us, const __half* ws, uint32_t mk[8],
                                                    float L[8][8], uint32_t& flags) {
    const bool sf16 = a.scale_f16 != 0;
    const int G = g.j0 / a.group;
    const int gl = a.group >> 3;
    uint8_t* cp = tb + ((size_t)(g.j0 >> 3) * (a.dk >> 3) + (g.i0 >> 3)) * (8 * BITS);
    uint8_t* sp = tb + he.scales + ((size_t)G * a.dk + g.i0) * (sf16 ? 2 : 4);
    Chunk<BITS> ch;
    load_chunk<BITS>(cp, ch);
    float s_old[8];
    load_scales8(sf16, sp, s_old);
    // the codes are unpacked row by row where needed (unused rows of an
    // inlined unpack are dropped), which keeps the live set to L or x plus q
    float x[8][8];
    bool nonfinite = false;
    {
      low_rank(a, g, us, ws, L);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float thr = __fmul_rn(a.lrb_eps, s_old[i]);
        float cf[8][8];
        unpack(ch, cf);
        uint32_t bits = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float shat = __fmul_rn(cf[i][j], s_old[i]);
          const float l = L[i][j];
          const bool m = fabsf(l) > thr;
          x[i][j] = m ? __fadd_rn(shat, l) : shat;
          bits |= ((uint32_t)(m && l > 0.f) << j) | ((uint32_t)(m && l < 0.f) << (8 + j));
          nonfinite = nonfinite || !(fabsf(x[i][j]) <= 3.4e38f);
        }
        // keep the flags as one integer per row (left to itself the compiler
        // carries 128 per-element lane masks in SGPRs until they are used)
        asm volatile("" : "+v"(bits));
        mk[i] = bits;
      }
    }
    if (nonfinite) flags |= kStatusNonfinite;

    // scale rule on x
    constexpr int qmax = (1 << (BITS - 1)) - 1;
    constexpr float qmaxf = (float)qmax;
    constexpr int lo = -(qmax + 1), hi = qmax;
    float s_new[8];
    const float trig_q = __fmul_rn(a.trigger, qmaxf);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float m = group_max_rt(absmax8(x[i]), gl);
      const float ratio = m / qmaxf;
      const float fresh = sf16 ? __half2float(__float2half_rn(ratio)) : ratio;
      if (a.smode == kScalePersistent) {
        const float thr = __fmul_rn(trig_q, s_old[i]);
        s_new[i] = (m > thr) ? fresh : s_old[i];
      } else {
        s_new[i] = fresh;
      }
      if (sf16 && __builtin_isinf(s_new[i])) flags |= kStatusScaleOverflow;
    }

    // RNE of the exact product x * RN(1/s'), clamped; BDR toward sign(L) on M,
    // with the unmerged value s_hat as the no-update reference (branch-free)
    int q[8][8];
    bool clipped = false;
    const float gate_k = __fadd_rn(0.5f, a.bdr_eps);
    const float lof = (float)lo, hif = (float)hi;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sn = s_new[i];
      const float inv = (sn == 0.f) ? 0.f : 1.0f / sn;
      const float gate = __fmul_rn(gate_k, sn);
      float cf[8][8];
      unpack(ch, cf);
      float over = -1.f;   // > 0 when a finite code left the range
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float yr = __fmul_rn(x[i][j], inv);
        const float t = __fsub_rn(__builtin_fmaf(x[i][j], inv, kMagic), kMagic);   // RNE(x inv) for |x inv| < 2^22
        float c = (fabsf(yr) < 4194304.f) ? t : yr;
        const bool fin = fabsf(yr) <= 3.4e38f;
        over = fmaxf(over, fin ? fmaxf(c - hif, lof - c) : -1.f);
        c = (c == c) ? fminf(fmaxf(c, lof), hif) : lof;   // a NaN product takes the low code
        const uint32_t mb = (mk[i] >> j) & 0x101u;
        const float sg = (a.bdr && sn > 0.f) ? ((mb & 1u) ? 1.f : ((mb & 0x100u) ? -1.f : 0.f)) : 0.f;
        const float r = __fmul_rn(cf[i][j], s_old[i]);
        const float val = __fmul_rn(c, sn);
        const bool rev = sg * __fsub_rn(val, r) < 0.f;   // the sign of a float difference is exact
        const float cand = fminf(fmaxf(c + sg, lof), hif);
        const float err = fabsf(__fsub_rn(x[i][j], __fmul_rn(cand, sn)));
        c = (rev && err <= gate && cand != c) ? cand : c;
        q[i][j] = (int)c;
      }
      clipped = clipped || over > 0.f;
    }
    if (clipped) flags |= kStatusClipped;
    Chunk<BITS> out;
    pack(q, out);
    store_chunk<BITS>(cp, out);
    if ((g.lc & (gl - 1)) == 0) store_scales8(sf16, sp, s_new);
  }

  // ------------------------------------------------------------ products with R
  // yt[c][i] = sum_j R_ij zt[c][j] for c < p
  static __device__ __forceinline__ void prod_rz(const StepArgs& a, const Geo& g, const float R[8][8], const MergeLds& S, int p) {
    const int zs = merge_zs(a.dv), ys = merge_ys(a.dk);
    const int C = a.merge_chunk;
    for (int c0 = 0; c0 < p; c0 += C) {
      const int nc = min(C, p - c0);
      for (int cc = 0; cc < nc; ++cc) {
        float z8[8];
        loadf8(S.zt + (size_t)(c0 + cc) * zs + g.j0, z8);
        float y8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float acc = __fmul_rn(R[i][0], z8[0]);
#pragma unroll
          for (int j = 1; j < 8; ++j) acc = __builtin_fmaf(R[i][j], z8[j], acc);
          y8[i] = col_lane_sum<CL>(acc);
        }
        if (g.lc == 0) storef8(S.part + ((size_t)g.wc * C + cc) * a.dk + g.i0, y8);
      }
      __syncthreads();
      for (int e = threadIdx.x; e < nc * a.dk; e += blockDim.x) {
        const int cc = e / a.dk, i = e - cc * a.dk;
        float s = S.part[(size_t)cc * a.dk + i];
        for (int w = 1; w < g.wcw; ++w) s = __fadd_rn(s, S.part[((size_t)w * C + cc) * a.dk + i]);
        S.yt[(size_t)(c0 + cc) * ys + i] = s;
      }
      __syncthreads();
    }
  }

  // zt[c][j] = sum_i R_ij yt[c][i] for c < p
  static __device__ __forceinline__ void prod_rty(const StepArgs& a, const Geo& g, const float R[8][8], const MergeLds& S, int p) {
    const int zs = merge_zs(a.dv), ys = merge_ys(a.dk);
    const bool writer = NB < 4 || ((g.lane >> 2) & 1) == 0;
    const int C = a.merge_chunk;
    for (int c0 = 0; c0 < p; c0 += C) {
      const int nc = min(C, p - c0);
      for (int cc = 0; cc < nc; ++cc) {
        float q8[8];
        loadf8(S.yt + (size_t)(c0 + cc) * ys + g.i0, q8);
        float z8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float acc = __fmul_rn(R[0][j], q8[0]);
#pragma unroll
          for (int i = 1; i < 8; ++i) acc = __builtin_fmaf(R[i][j], q8[i], acc);
          z8[j] = acc;
        }
        xtree<NB>(z8, g.lane);
#pragma unroll
        for (int s = 0; s < NSLOT; ++s)
          if (writer) S.part[((size_t)g.wr * C + cc) * a.dv + g.j0 + xtree_col<NB>(s, g.lane)] = z8[s];
      }
      __syncthreads();
      for (int e = threadIdx.x; e < nc * a.dv; e += blockDim.x) {
        const int cc = e / a.dv, j = e - cc * a.dv;
        float s = S.part[(size_t)cc * a.dv + j];
        for (int w = 1; w < g.wrw; ++w) s = __fadd_rn(s, S.part[((size_t)w * C + cc) * a.dv + j]);
        S.zt[(size_t)(c0 + cc) * zs + j] = s;
      }
      __syncthreads();
    }
  }

  // ------------------------------------------------------------ small dense pieces
  // gram[a][b] = sum_i X[a][i] X[b][i] (X column-major: column c at xt + c * xs).
  // Wavefront w sums rows [w*m/nw, (w+1)*m/nw) for the pairs its lanes own;
  // the per-wavefront partials are then added in wavefront order.
  static __device__ __forceinline__ void gram(const Geo& g, const float* xt, int xs, int m, int p, float* gm,
                                              float* part) {
    const int npairs = p * (p + 1) / 2;
    const int rows = (m + g.nw - 1) / g.nw;
    const int r0 = g.wave * rows, r1 = min(m, r0 + rows);
    for (int pi = g.lane; pi < npairs; pi += 64) {
      int ca, cb;
      tri_pair(pi, p, ca, cb);
      const float* xa = xt + (size_t)ca * xs;
      const float* xb = xt + (size_t)cb * xs;
      float s0 = 0.f, s1 = 0.f;
      int r = r0;
      if ((rows & 3) == 0) {
        // 16-byte reads: the row stride and the wavefront's first row are
        // multiples of 4 floats
        for (; r + 3 < r1; r += 4) {
          const float4 a4 = *reinterpret_cast<const float4*>(xa + r);
          const float4 b4 = *reinterpret_cast<const float4*>(xb + r);
          s0 = __builtin_fmaf(a4.x, b4.x, s0);
          s1 = __builtin_fmaf(a4.y, b4.y, s1);
          s0 = __builtin_fmaf(a4.z, b4.z, s0);
          s1 = __builtin_fmaf(a4.w, b4.w, s1);
        }
      }
      for (; r + 1 < r1; r += 2) {
        s0 = __builtin_fmaf(xa[r], xb[r], s0);
        s1 = __builtin_fmaf(xa[r + 1], xb[r + 1], s1);
      }
      if (r < r1) s0 = __builtin_fmaf(xa[r], xb[r], s0);
      part[g.wave * kTri + pi] = __fadd_rn(s0, s1);
    }
    __syncthreads();
    for (int pi = threadIdx.x; pi < npairs; pi += blockDim.x) {
      float s = part[pi];
      for (int w = 1; w < g.nw; ++w) s = __fadd_rn(s, part[w * kTri + pi]);
      int ca, cb;
      tri_pair(pi, p, ca, cb);
      gm[ca * kSm + cb] = s;
      gm[cb * kSm + ca] = s;
    }
    __syncthreads();
  }

  // G = L L^T for the p x p Gram matrix in gm (row stride kSm), p <= P. Lane i
  // holds row i; column k of L reaches the other lanes through readlane.
  // Writes L (rows, stride kMaxCap; only the entries left of the diagonal
  // matter) to lt and 1/L_kk to dinv (0 for a dropped column).
  template <int P>
  static __device__ __forceinline__ void cholesky(int i, int p, const float* gm, float* dinv, float* lt) {
    float row[P];
#pragma unroll
    for (int c = 0; c < P; ++c) row[c] = (i < p && c < p) ? gm[i * kSm + c] : 0.f;
    const float gii = (i < p) ? gm[i * kSm + i] : 0.f;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const float piv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row[k]), k));
      const float gkk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gii), k));
      const bool live = piv > 1e-6f * gkk && piv > 0.f;
      // 1/sqrt to about an ulp is plenty: the second pass of CholeskyQR2
      // removes what the first leaves
      const float di = live ? __builtin_amdgcn_rsqf(piv) : 0.f;
      // lanes i > k get L_ik; the other lanes only touch the upper
      // triangle, which is never read (the diagonal is kept as 1/d)
      const float lik = __fmul_rn(row[k], di);
      row[k] = lik;
      if (i == 0) dinv[k] = di;
#pragma unroll
      for (int j = k + 1; j < P; ++j) {
        const float ljk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lik), j));
        row[j] = __fsub_rn(row[j], __fmul_rn(lik, ljk));
      }
    }
    if (i < p) {
#pragma unroll
      for (int c = 0; c < P; c += 4)
        *reinterpret_cast<float4*>(lt + i * kMaxCap + c) = make_float4(row[c], row[c + 1], row[c + 2], row[c + 3]);
    }
  }

  // In place: X <- X L^-T with G = X^T X = L L^T (Cholesky), `passes` times
  // (2: CholeskyQR2). A column whose remaining norm is below 1e-3 of its own
  // (pivot below 1e-6 of its Gram diagonal) gets 1/diag = 0: it drops out.
  static __device__ __forceinline__ void orth(const Geo& g, float* xt, int xs, int m, int p, const MergeLds& S,
                                              int passes) {
    float* dinv = S.misc + kMiscDinv;
    float* lt = S.h1;    // L, row stride kMaxCap (16-byte aligned rows); free outside the Jacobi
    for (int pass = 0; pass < passes; ++pass) {
      gram(g, xt, xs, m, p, S.g, S.part);
      if (g.wave == 0) {
        // p rounded up to a multiple of 4 or 8 fixes the loop bounds; the
        // padded columns are zero and drop out like any dependent column
        if (p <= 8) cholesky<8>(g.lane, p, S.g, dinv, lt);
        else if (p <= 16) cholesky<16>(g.lane, p, S.g, dinv, lt);
        else if (p <= 20) cholesky<20>(g.lane, p, S.g, dinv, lt);
        else if (p <= 24) cholesky<24>(g.lane, p, S.g, dinv, lt);
        else cholesky<32>(g.lane, p, S.g, dinv, lt);
      }
      __syncthreads();
      // forward substitution per row of X, in registers
      for (int r = threadIdx.x; r < m; r += blockDim.x) {
        float v[kMaxCap];
#pragma unroll
        for (int c = 0; c < kMaxCap; ++c) {
          if (c < p) {
            float acc = xt[(size_t)c * xs + r];
#pragma unroll
            for (int j0 = 0; j0 < c; j0 += 4) {
              const float4 l4 = *reinterpret_cast<const float4*>(lt + c * kMaxCap + j0);
              acc = __fsub_rn(acc, __fmul_rn(l4.x, v[j0]));
              if (j0 + 1 < c) acc = __fsub_rn(acc, __fmul_rn(l4.y, v[j0 + 1]));
              if (j0 + 2 < c) acc = __fsub_rn(acc, __fmul_rn(l4.z, v[j0 + 2]));
              if (j0 + 3 < c) acc = __fsub_rn(acc, __fmul_rn(l4.w, v[j0 + 3]));
            }
            v[c] = __fmul_rn(acc, dinv[c]);
            xt[(size_t)c * xs + r] = v[c];
          }
        }
      }
      __syncthreads();
    }
  }

  // Partner of index x in round r of the round-robin schedule for P (even)
  // players: (P-1, r) and (r+k, r-k) mod (P-1) for k = 1 .. P/2-1.
  static __device__ __forceinline__ int rr_partner(int x, int r, int P) {
    if (x == P - 1) return r;
    if (x == r) return P - 1;
    int y = 2 * r - x;
    y = (y < 0) ? y + (P - 1) : y;
    return (y >= P - 1) ? y - (P - 1) : y;
  }

  // Cyclic Jacobi on the symmetric p x p matrix in S.h0, all threads. Per
  // round, the P/2 disjoint rotations of the round-robin schedule: one thread
  // per rotation finds its angle and publishes J_xx, J_yx for both indices,
  // then H <- J^T H J and V <- V J go element-wise into the other buffer. On
  // return H points at the eigenvalues (diagonal) and V at the eigenvectors
  // (columns).
  static __device__ __forceinline__ void jacobi(const Geo& g, int p, float*& H, float*& V, float*& Hn, float*& Vn,
                                                const MergeLds& S) {
    for (int e = threadIdx.x; e < p * p; e += blockDim.x) {
      const int i = e / p, j = e - i * p;
      V[i * kSm + j] = (i == j) ? 1.f : 0.f;
    }
    const int P = (p + 1) & ~1;
    float* flag = S.misc + kMiscFlag;
    float* rot = S.misc + kMiscRot;   // [kMaxCap][2]: J_xx, J_(partner, x)
    __syncthreads();
    for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
      if (g.wave == 0) {
        float off = 0.f, dia = 0.f;
        for (int e = g.lane; e < p * p; e += 64) {
          const int i = e / p, j = e - i * p;
          const float h = H[i * kSm + j];
          if (i == j) dia = __builtin_fmaf(h, h, dia);
          else off = __builtin_fmaf(h, h, off);
        }
        off = wave_sum(off);
        dia = wave_sum(dia);
        // an off-diagonal norm of 1e-2 of the diagonal's leaves eigenvector
        // errors of that order, whose effect on the rank-k error is of second
        // order (about 1e-4 relative): on the GLA workload's residuals the
        // excess over the Eckart-Young optimum is the same as with a 1e-4
        // stop, one sweep earlier
        if (g.lane == 0) flag[0] = (off <= 1e-4f * dia) ? 1.f : 0.f;
      }
      __syncthreads();
      if (flag[0] != 0.f) break;
      for (int round = 0; round < P - 1; ++round) {
        if ((int)threadIdx.x < p) {
          const int x = threadIdx.x, y = rr_partner(x, round, P);
          if (x < y) {
            float c = 1.f, sn = 0.f;
            if (y < p) {
              const float haa = H[x * kSm + x], hbb = H[y * kSm + y], hab = H[x * kSm + y];
              if (hab != 0.f) {
                // the angle to about an ulp: the rotations stay orthogonal to that order
                const float th = (hbb - haa) * (0.5f * __builtin_amdgcn_rcpf(hab));
                const float at = fabsf(th);
                const float t = (at > 1e18f) ? 0.5f * __builtin_amdgcn_rcpf(th)
                                             : copysignf(__builtin_amdgcn_rcpf(at + __builtin_amdgcn_sqrtf(th * th + 1.f)), th);
                c = __builtin_amdgcn_rsqf(t * t + 1.f);
                sn = t * c;
              }
            }
            rot[2 * x] = c;
            rot[2 * x + 1] = -sn;       // J_(y, x) = -s for the lower index
            if (y < p) {
              rot[2 * y] = c;
              rot[2 * y + 1] = sn;      // J_(x, y) = s
            }
          } else if (y >= p) {
            rot[2 * x] = 1.f;           // paired with the padding player
            rot[2 * x + 1] = 0.f;
          }
        }
        __syncthreads();
        for (int e = threadIdx.x; e < p * p; e += blockDim.x) {
          const int i = e / p, j = e - i * p;
          int pi = rr_partner(i, round, P), pj = rr_partner(j, round, P);
          pi = (pi < p) ? pi : i;
          pj = (pj < p) ? pj : j;
          const float2 ri = *reinterpret_cast<const float2*>(rot + 2 * i);
          const float2 rj = *reinterpret_cast<const float2*>(rot + 2 * j);
          Hn[i * kSm + j] = ri.x * (rj.x * H[i * kSm + j] + rj.y * H[i * kSm + pj]) +
                            ri.y * (rj.x * H[pi * kSm + j] + rj.y * H[pi * kSm + pj]);
          Vn[i * kSm + j] = rj.x * V[i * kSm + j] + rj.y * V[i * kSm + pj];
        }
        __syncthreads();
        float* t = H; H = Hn; Hn = t;
        t = V; V = Vn; Vn = t;
      }
    }
  }

  // ------------------------------------------------------------ the kernel body
  static __device__ __forceinline__ void run(const StepArgs& a) {
    extern __shared__ float lds[];
    const int tile = blockIdx.x;
    const int bb = tile / a.H, h = tile - bb * a.H;
    const HeadEntry he = head_entry(a, h);
    uint8_t* tb = a.tiles + (size_t)bb * a.batch_stride + he.head_offset;
    const Geo g = geo(a);
    MergeLds S;
    S.zt = lds;
    S.yt = S.zt + (size_t)a.cap * merge_zs(a.dv);
    S.part = S.yt + (size_t)a.cap * merge_ys(a.dk);
    S.g = S.part + merge_part_floats(a.dk, a.dv, g.wrw, g.wcw, a.merge_chunk);
    S.h0 = S.g + kMaxCap * kSm;
    S.h1 = S.h0 + kMaxCap * kSm;
    S.v0 = S.h1 + kMaxCap * kSm;
    S.v1 = S.v0 + kMaxCap * kSm;
    S.misc = S.v1 + kMaxCap * kSm;

    uint32_t flags = 0;
    // the bypass factors go through LDS (the basis areas are free until the
    // subspace iteration); L is formed once from them and kept for R
    __half* us = reinterpret_cast<__half*>(S.yt);
    __half* ws = reinterpret_cast<__half*>(S.zt);
    stage_bypass(a, he, tb, us, ws);
    uint32_t mk[8];
    float R[8][8];   // L, kept through the requantization
    switch (he.bits) {
      case 4: requantize<4>(a, he, tb, g, us, ws, mk, R, flags); break;
      case 6: requantize<6>(a, he, tb, g, us, ws, mk, R, flags); break;
      default: requantize<8>(a, he, tb, g, us, ws, mk, R, flags); break;
    }
    // the residual R = L on the elements that stayed in the bypass
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((mk[i] >> j) & 0x101u) R[i][j] = 0.f;
    __syncthreads();   // the staging area becomes the bases

    const int p = a.n;
    const int k = min(a.lrb_k, p);
    __half* U = reinterpret_cast<__half*>(tb + he.bypass_u);
    __half* W = reinterpret_cast<__half*>(tb + he.bypass_w);
    const int zs = merge_zs(a.dv), ys = merge_ys(a.dk);
    float* H = S.h0;
    float* Hn = S.h1;
    float* V = S.v0;
    float* Vn = S.v1;
    if (k > 0) {
      // start from the bypass's right factors (all of W is read before any of it is rewritten)
      for (int e = threadIdx.x; e < p * a.dv; e += blockDim.x) {
        const int c = e / a.dv, j = e - c * a.dv;
        S.zt[(size_t)c * zs + j] = __half2float(W[(size_t)c * a.dv + j]);
      }
      __syncthreads();
      const int iters = (p >= 4 * k + 4) ? kMergeItersWide : kMergeItersNarrow;
      // Z needs no orthonormalisation of its own: span(R Z) does not depend
      // on the basis of span(Z), and Q = orth(R Z) keeps the numbers in range
      for (int it = 0; it < iters; ++it) {
        prod_rz(a, g, R, S, p);
        // one CholeskyQR pass keeps an intermediate basis well conditioned;
        // the final one, which the factors are built from, gets two
        orth(g, S.yt, ys, a.dk, p, S, it + 1 < iters ? 1 : 2);
        prod_rty(a, g, R, S, p);
      }
      // Rayleigh-Ritz: B = Q^T R = Z^T, B B^T = Z^T Z
      gram(g, S.zt, zs, a.dv, p, H, S.part);
      jacobi(g, p, H, V, Hn, Vn, S);
      // order of the eigenvalues, largest first (ties by index)
      int* order = reinterpret_cast<int*>(S.misc + kMiscOrder);
      float* sroot = S.misc + kMiscSroot;
      if (g.wave == 0 && g.lane < p) {
        // a NaN eigenvalue sorts last, so the ranks stay a permutation
        auto key = [](float v) { return v == v ? v : -INFINITY; };
        const float lam = key(H[g.lane * kSm + g.lane]);
        int rank = 0;
        for (int j = 0; j < p; ++j) {
          const float lj = key(H[j * kSm + j]);
          rank += (lj > lam || (lj == lam && j < g.lane)) ? 1 : 0;
        }
        order[rank] = g.lane;
      }
      __syncthreads();
      if (g.wave == 0 && g.lane < k) {
        const float lam = H[order[g.lane] * kSm + order[g.lane]];
        sroot[g.lane] = lam > 0.f ? __fsqrt_rn(__fsqrt_rn(lam)) : 0.f;   // sigma^(1/2)
      }
      __syncthreads();
      // sign of each U column: its largest-magnitude entry (first on ties) is positive
      float* sgn = S.misc + kMiscSign;
      for (int mcol = g.wave; mcol < k; mcol += g.nw) {
        const int oc = order[mcol];
        float best = -1.f, bval = 0.f;
        int bidx = 0x7fffffff;
        for (int i = g.lane; i < a.dk; i += 64) {
          float u = 0.f;
          for (int c = 0; c < p; ++c) u = __builtin_fmaf(S.yt[(size_t)c * ys + i], V[c * kSm + oc], u);
          // judged on the value as stored (binary16, whose rounding is odd-symmetric)
          const float au = fabsf(__half2float(__float2half_rn(u * sroot[mcol])));
          if (au > best || (au == best && i < bidx)) { best = au; bval = u; bidx = i; }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
          const float ob = __shfl_xor(best, m, 64), ov = __shfl_xor(bval, m, 64);
          const int oi = __shfl_xor(bidx, m, 64);
          if (ob > best || (ob == best && oi < bidx)) { best = ob; bval = ov; bidx = oi; }
        }
        if (g.lane == 0) sgn[mcol] = (bval < 0.f) ? -1.f : 1.f;
      }
      __syncthreads();
      // U_k S^1/2 = Q V_k S^1/2 and V_k S^1/2 = Z V_k S^-1/2, rounded to binary16
      for (int e = threadIdx.x; e < k * a.dk; e += blockDim.x) {
        const int mcol = e / a.dk, i = e - mcol * a.dk;
        const int oc = order[mcol];
        float u = 0.f;
        for (int c = 0; c < p; ++c) u = __builtin_fmaf(S.yt[(size_t)c * ys + i], V[c * kSm + oc], u);
        U[(size_t)mcol * a.dk + i] = __float2half_rn(sgn[mcol] * (u * sroot[mcol]));
      }
      for (int e = threadIdx.x; e < k * a.dv; e += blockDim.x) {
        const int mcol = e / a.dv, j = e - mcol * a.dv;
        const int oc = order[mcol];
        float w = 0.f;
        for (int c = 0; c < p; ++c) w = __builtin_fmaf(S.zt[(size_t)c * zs + j], V[c * kSm + oc], w);
        const float sr = sroot[mcol];
        W[(size_t)mcol * a.dv + j] = __float2half_rn(sr > 0.f ? sgn[mcol] * (w / sr) : 0.f);
      }
    }
    // the columns past k are empty
    for (int e = threadIdx.x; e < (a.cap - k) * a.dk; e += blockDim.x)
      U[(size_t)k * a.dk + e] = __float2half_rn(0.f);
    for (int e = threadIdx.x; e < (a.cap - k) * a.dv; e += blockDim.x)
      W[(size_t)k * a.dv + e] = __float2half_rn(0.f);

    if (any_lane(flags != 0)) {
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) flags |= (uint32_t)__shfl_xor((int)flags, m, 64);
      if (g.lane == 0) atomicOr(a.status, flags);
    }
    if (tile == 0 && threadIdx.x == 0) *a.hdr_n = a.lrb_k;
  }
};

template <int CL>
__global__ __launch_bounds__(512) void merge_kernel(StepArgs a) {
  Merge<CL>::run(a);
}

DecodeFn merge_kernel_for(int cl) {
  switch (cl) {
    case 4: return merge_kernel<4>;
    case 8: return merge_kernel<8>;
    default: return merge_kernel<16>;
  }
}

}  // namespace rsq
