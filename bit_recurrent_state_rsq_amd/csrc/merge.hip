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
// The rank-k approximation works on the Gram matrix of R's narrower side:
// C = R^T R (d_v x d_v) when d_v <= d_k, else C = R R^T. C is formed once on
// the matrix cores: R is scaled by a power of two into binary16 range and
// split into a high and a low binary16 part, and the three products hi*hi,
// hi*lo and lo*hi accumulate in float32 (the dropped lo*lo term is below
// 2^-22 of each product). A fixed number of subspace iterations
//   Q <- orth(C Q)   (or orth(C C Q) while the basis stays well conditioned)
// start from the bypass's own factors on that side, which span the row or
// column space of L (an all-zero start column gets a fixed +-1 pattern), with
// C Q again on split binary16 matrix cores. orth is CholeskyQR: wavefront 0
// forms the basis's Gram matrix on the matrix cores, factors it and inverts
// the factor with cross-lane reads, and every thread then applies the inverse
// to its rows; a second pass (CholeskyQR2) follows when the first one's
// condition estimate is above 20. Rayleigh-Ritz then diagonalises the p x p
// matrix Q^T C Q by cyclic Jacobi (in one wavefront when p <= 16); its top k
// eigenpairs (sigma^2, v) give the narrow-side singular vectors Q v, and the
// other side's R (Q v) / sigma comes from R, which every lane still holds in
// registers in the decode kernel's 8x8-chunk layout.
//
// Working on C squares R's condition number. A direction of R whose singular
// value is below a few percent of the largest sinks, in C Q, below the
// CholeskyQR pivot threshold and can be lost; that costs accuracy only when
// fewer than k directions are stronger, so that the kept rank reaches down to
// such a weak one.
#include <algorithm>

#include "rsq_kernels.hpp"
#include "lane_ops.hpp"

namespace rsq {

// Subspace iterations (products with C = R^T R): each one shrinks the error
// of the rank-k subspace by about (sigma_(p+1) / sigma_k)^2, so a narrow
// bypass (few columns per kept rank) needs more of them. With the warm start
// these bring the Frobenius error within 2e-4 of the Eckart-Young optimum on
// the workloads' residuals.
constexpr int kMergeItersWide = 4;    // p >= 8k + 8
constexpr int kMergeItersMid = 5;     // p >= 3k + 4
constexpr int kMergeItersNarrow = 12;
// A basis whose last condition estimate is at most this takes two products
// with C before it is orthonormalised again (the condition number grows by
// at most the product's); on the workloads' residuals 128 leaves the
// Eckart-Young excess where 8 had it and saves most tiles an orthonormalisation
constexpr float kDoubleKappa = 128.f;
constexpr int kJacobiSweeps = 12;  // upper bound; stops once the off-diagonal part is negligible
constexpr int kSm = kMaxCap + 1;   // row stride of the small p x p matrices
constexpr int kWs = kMaxCap + 4;   // row stride of the Gram / Cholesky scratch (16-byte rows)
constexpr int kWsFloats = (2 * kMaxCap + 1) * kWs;   // L's rows, a row of 1/diagonal, L^-1's rows
constexpr int kQScale = 12;        // an orthonormal basis times 2^12 fits binary16 with room for its low part
// misc block layout (floats)
constexpr int kMiscOrder = 0, kMiscSroot = kMaxCap, kMiscSign = 2 * kMaxCap, kMiscFlag = 3 * kMaxCap,
              kMiscWave = 3 * kMaxCap + 4,   // [8] maxima, [8] non-finite flags per wavefront
              kMiscJac = 3 * kMaxCap + 20,   // [2][8][2] Jacobi off-diagonal / diagonal partial sums
              kMiscSinv = 3 * kMaxCap + 52,  // [kMaxCap] sigma^-1/2
              kMiscOrth = 4 * kMaxCap + 52,  // condition estimate and scale exponent of the last orth pass
              kMiscFloats = 7 * kMaxCap;

typedef _Float16 h4v __attribute__((ext_vector_type(4)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

__host__ __device__ inline int merge_zs(int dv) { return dv + 4; }
__host__ __device__ inline int merge_ys(int dk) { return dk + 4; }

// floats of the partial-sum area of the closing products with R
__host__ __device__ inline size_t merge_part_floats(int dk, int dv, int wrw, int wcw, int chunk) {
  return (size_t)chunk * (size_t)(wcw * dk > wrw * dv ? wcw * dk : wrw * dv);
}

// LDS carve-up of the merge kernel, in floats from the start of the dynamic
// area (X and C in halves). One area is shared by phases that never overlap
// in time; only `misc` lies outside it:
//   staging       the bypass factors (binary16)
//   phase B       X split: binary16 high and low planes, column-major, K + 8 halves per column
//   C             the split Gram matrix (row-major, N + 8 halves per row): kept
//                 through phase C, or (`creg`) only until every wavefront has
//                 loaded its rows' MFMA fragments into registers
//   phase C       q, y (bases, column-major, N + 4 floats per column), the Gram /
//                 Cholesky scratch (after C when C stays)
//   phase D       q (the final basis), the Jacobi buffers and rotations, the
//                 closing products' bases and partial sums
// `creg` holds when at most 8 columns are kept (the basis then has at most 16
// columns, one MFMA column block) and every wavefront owns at most two of
// C's 16-row blocks.
struct MergeLayout {
  int N, K, pc;       // narrow side, wide side, basis columns (a multiple of 16)
  bool right;         // N = d_v: C = R^T R (else C = R R^T)
  bool creg;          // C's fragments live in registers during the iteration
  size_t xh, xl;      // split X (halves)
  size_t ch, cl;      // split C (halves)
  size_t q, y, ws;    // bases; the Gram / Cholesky scratch
  size_t h0, h1, v0, v1, rot;   // Jacobi: H, V (double buffered), rotations [2][kMaxCap][4]
  size_t zt, yt, part;   // closing products
  size_t misc, total;
};

__host__ __device__ inline MergeLayout merge_layout(int dk, int dv, int wrw, int wcw, int cap, int k, int chunk) {
  MergeLayout L;
  L.right = dv <= dk;
  L.N = L.right ? dv : dk;
  L.K = L.right ? dk : dv;
  const int nw = wrw * wcw;
  L.creg = k <= 8 && ((L.N / 16) + nw - 1) / nw <= 2;
  L.pc = L.creg ? 16 : (cap + 15) & ~15;
  const size_t bs = (size_t)L.pc * (L.N + 4);
  const size_t csz = (size_t)L.N * (L.N + 8);   // two binary16 planes = one float per element
  const size_t stage = ((size_t)cap * (dk + dv) + 1) / 2;
  const size_t xsz = (size_t)L.N * (L.K + 8);
  L.xh = 0;
  L.xl = (size_t)L.N * (L.K + 8);
  L.q = 0;
  L.y = bs;
  const size_t c0 = L.creg ? 0 : 2 * bs;          // C (floats)
  L.ch = 2 * c0;
  L.cl = L.ch + (size_t)L.N * (L.N + 8);
  L.ws = L.creg ? 2 * bs : 2 * bs + csz;
  L.h0 = 2 * bs;
  L.h1 = L.h0 + kMaxCap * kSm;
  L.v0 = L.h1 + kMaxCap * kSm;
  L.v1 = L.v0 + kMaxCap * kSm;
  L.rot = L.v1 + kMaxCap * kSm;
  L.zt = L.rot + 8 * kMaxCap;
  L.yt = L.zt + (size_t)cap * merge_zs(dv);
  L.part = L.yt + (size_t)cap * merge_ys(dk);
  const size_t phase_c = L.ws + kWsFloats;
  const size_t phase_d = L.part + merge_part_floats(dk, dv, wrw, wcw, chunk);
  size_t u = stage;
  u = u > xsz ? u : xsz;
  u = u > c0 + csz ? u : c0 + csz;
  u = u > phase_c ? u : phase_c;
  u = u > phase_d ? u : phase_d;
  L.misc = (u + 3) & ~size_t(3);
  L.total = L.misc + kMiscFloats;
  return L;
}

size_t merge_lds_floats(int dk, int dv, int wrw, int wcw, int cap, int k, int chunk) {
  return merge_layout(dk, dv, wrw, wcw, cap, k, chunk).total;
}

// the closing products' view of the LDS (the register products with R)
struct MergeLds {
  float* zt;    // [cap][zs]       right vectors, column c at zt + c * zs
  float* yt;    // [cap][ys]       left vectors
  float* part;  // [stripes][chunk][rows]  per-wavefront-stripe partial sums
};

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

// sum or max over the 64 lanes, the same value in every lane: within each
// 16-lane row by DPP (quad permutes xor 1 and xor 2, half-row mirror, row
// mirror), then rows 0 and 2 into rows 1 and 3 (row_bcast15) and lane 31 into
// rows 2 and 3 (row_bcast31); lane 63 holds the total. No LDS round trip.
template <int CTRL, int ROWS, bool SUM>
__device__ __forceinline__ float dpp_step(float v) {
  const int idn = __float_as_int(SUM ? 0.f : -INFINITY);   // rows left out keep the operation's identity
  const float x = __int_as_float(__builtin_amdgcn_update_dpp(idn, __float_as_int(v), CTRL, ROWS, 0xF, false));
  return SUM ? __fadd_rn(v, x) : fmaxf(v, x);
}

template <bool SUM>
__device__ __forceinline__ float wave_reduce(float v) {
  v = dpp_step<0xB1, 0xF, SUM>(v);    // quad_perm [1, 0, 3, 2]
  v = dpp_step<0x4E, 0xF, SUM>(v);    // quad_perm [2, 3, 0, 1]
  v = dpp_step<0x141, 0xF, SUM>(v);   // row_half_mirror
  v = dpp_step<0x140, 0xF, SUM>(v);   // row_mirror
  v = dpp_step<0x142, 0xA, SUM>(v);   // row_bcast15 into rows 1 and 3
  v = dpp_step<0x143, 0xC, SUM>(v);   // row_bcast31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_sum(float v) { return wave_reduce<true>(v); }

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lane J of each 16-lane row, to every lane of the row (DPP row_newbcast).
template <int J>
__device__ __forceinline__ float bc16(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + J, 0xF, 0xF, true));
}
// acc += (lane J's src) m in one instruction (v_fmac_f32 with the broadcast on
// src). The caller makes sure that src was not written by the two cycles
// before (the DPP read hazard): see dpp_ready.
template <int J>
__device__ __forceinline__ void fmac_bc16(float& acc, float src, float m) {
  asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(src), "v"(m), "n"(J));
}
// two wait states after v was written, before a DPP instruction reads it
__device__ __forceinline__ void dpp_ready(float& v) { asm volatile("s_nop 1" : "+v"(v)); }

// Cholesky of a p x p Gram matrix (p <= 16) in one wavefront, lane i holding
// row i: step K broadcasts the pivot and L's column K within the 16-lane row
// (no scalar round trip), and each update is one fused multiply-add.
template <int P8, int J>
__device__ __forceinline__ void chol16_upd(float (&row)[P8], float lik, float nlik) {
  if constexpr (J < P8) {
    fmac_bc16<J>(row[J], lik, nlik);   // row_J -= L_Jk L_lk
    chol16_upd<P8, J + 1>(row, lik, nlik);
  }
}
template <int P8, int K>
__device__ __forceinline__ void chol16(float (&row)[P8], float gii, float& dmine, int l) {
  if constexpr (K < P8) {
    dpp_ready(row[K]);
    const float piv = bc16<K>(row[K]);
    const float gkk = bc16<K>(gii);
    const bool live = piv > 1e-6f * gkk && piv > 0.f;
    // 1/sqrt to about an ulp: the next pass (or CholeskyQR2) removes what this one leaves
    const float di = live ? __builtin_amdgcn_rsqf(piv) : 0.f;
    float lik = __fmul_rn(row[K], di);
    row[K] = lik;
    if (l == K) dmine = di;
    const float nlik = -lik;
    dpp_ready(lik);
    chol16_upd<P8, K + 1>(row, lik, nlik);
    chol16<P8, K + 1>(row, gii, dmine, l);
  }
}
// L^-1 by columns (lane l forms column l), the same way: x_I = (I == l ? 1 :
// -sum_{t<I} L_It x_t) / L_II, with L_It (lane I's row[t]) and 1/L_II broadcast
template <int P8, int I, int T>
__device__ __forceinline__ void linv16_sum(const float (&row)[P8], const float (&x)[P8], float (&s4)[4]) {
  if constexpr (T < I) {
    fmac_bc16<I>(s4[T & 3], row[T], x[T]);
    linv16_sum<P8, I, T + 1>(row, x, s4);
  }
}
template <int P8, int I>
__device__ __forceinline__ void linv16(const float (&row)[P8], float dmine, float (&x)[P8], int l, float* Mi, int ws) {
  if constexpr (I < P8) {
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
    linv16_sum<P8, I, 0>(row, x, s4);
    const float su = __fadd_rn(__fadd_rn(s4[0], s4[1]), __fadd_rn(s4[2], s4[3]));
    const float di = bc16<I>(dmine);
    x[I] = (I == l) ? di : ((I < l) ? 0.f : -__fmul_rn(di, su));
    if (l < P8) Mi[I * ws + l] = x[I];
    linv16<P8, I + 1>(row, dmine, x, l, Mi, ws);
  }
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
  // U and W (binary16) of the tile into LDS, column-major like in memory (W
  // right after U): every thread issues up to two 16-byte loads before it
  // stores any of them
  static __device__ __forceinline__ void stage_bypass(const StepArgs& a, const HeadEntry& he, const uint8_t* tb,
                                                      __half* us) {
    const uint4* U = reinterpret_cast<const uint4*>(tb + he.bypass_u);
    const uint4* W = reinterpret_cast<const uint4*>(tb + he.bypass_w);
    const int nu = a.n * a.dk / 8, tot = nu + a.n * a.dv / 8;   // 16-byte pieces
    uint4* dst = reinterpret_cast<uint4*>(us);
    const int nt = blockDim.x;
    for (int e = threadIdx.x; e < tot; e += 2 * nt) {
      const int e2 = e + nt;
      // (no branch between the loads and the stores: a thread without a
      // second piece loads and stores its first one twice)
      const bool two = e2 < tot;
      const int f = two ? e2 : e;
      const uint4* p0 = (e < nu) ? U + e : W + (e - nu);
      const uint4* p1 = (f < nu) ? U + f : W + (f - nu);
      const uint4 v0 = *p0, v1 = *p1;
      dst[e] = v0;
      dst[f] = v1;
    }
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
  // The lane's codes and step sizes are loaded before the bypass factors are
  // staged, so that both reads share one round trip to memory.
  template <int BITS>
  static __device__ __forceinline__ void requantize(const StepArgs& a, const HeadEntry& he, uint8_t* tb, const Geo& g,
                                                    __half* us, __half* ws, uint32_t mk[8],
                                                    float L[8][8], uint32_t& flags) {
    const bool sf16 = a.scale_f16 != 0;
    const int G = g.j0 / a.group;
    const int gl = a.group >> 3;
    uint8_t* cp = tb + ((size_t)(g.j0 >> 3) * (a.dk >> 3) + (g.i0 >> 3)) * (8 * BITS);
    uint8_t* sp = tb + he.scales + ((size_t)G * a.dk + g.i0) * (sf16 ? 2 : 4);
    Chunk<BITS> ch;
    load_chunk<BITS>(cp, ch);
    // the step sizes' raw words: converted after the staging, so that no wait
    // for them comes before its loads
    uint4 sraw[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
    sraw[0] = *reinterpret_cast<const uint4*>(sp);
    if (!sf16) sraw[1] = *reinterpret_cast<const uint4*>(sp + 16);
    stage_bypass(a, he, tb, us);
    float s_old[8];
    {
      const uint32_t w[8] = {sraw[0].x, sraw[0].y, sraw[0].z, sraw[0].w, sraw[1].x, sraw[1].y, sraw[1].z, sraw[1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        s_old[i] = sf16 ? __half2float(__ushort_as_half((uint16_t)((i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu))))
                        : __uint_as_float(w[i]);
    }
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

  // ------------------------------------------------------------ the factorisation on the matrix cores
  static __device__ __forceinline__ float wave_max(float v) { return wave_reduce<false>(v); }

  // e with m 2^e in [2^14, 2^15) for a finite m > 0 (binary16's largest finite is 65504)
  static __device__ __forceinline__ int fit_exp(float m) {
    int ex;
    frexpf(m, &ex);
    return 15 - ex;
  }

  // v 2^e as binary16 high and low parts: hi = RN16(x), lo = RN16(x - hi), the
  // difference being exact in float32
  static __device__ __forceinline__ void split8(const float v[8], int e, h8v& hi, h8v& lo) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float x = ldexpf(v[t], e);
      const _Float16 h = (_Float16)x;
      hi[t] = h;
      lo[t] = (_Float16)__fsub_rn(x, (float)h);
    }
  }

  // X from the lane's chunk of R, times 2^e and split. X is R (its columns are
  // R's columns) when d_v <= d_k, else R^T; K is X's row index.
  static __device__ __forceinline__ void write_x(const Geo& g, const MergeLayout& ML, const float R[8][8], int e,
                                                 _Float16* xh, _Float16* xl) {
    const size_t xs = (size_t)ML.K + 8;
    if (ML.right) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = R[t][c];
        h8v hi, lo;
        split8(v, e, hi, lo);
        *reinterpret_cast<h8v*>(xh + (size_t)(g.j0 + c) * xs + g.i0) = hi;
        *reinterpret_cast<h8v*>(xl + (size_t)(g.j0 + c) * xs + g.i0) = lo;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        h8v hi, lo;
        split8(R[r], e, hi, lo);
        *reinterpret_cast<h8v*>(xh + (size_t)(g.i0 + r) * xs + g.j0) = hi;
        *reinterpret_cast<h8v*>(xl + (size_t)(g.i0 + r) * xs + g.j0) = lo;
      }
    }
  }

  // C = X^T X (N x N) in 32 x 32 blocks, block b = J1 * (N/32) + J2 holding
  // C[J1 block rows][J2 block columns]; wavefront w takes blocks w, w + nw, ...
  // (at most four: N = 128 implies at least four wavefronts). Lane l of a block
  // reads X's columns J*32 + l%32 at rows 16 s + 8 (l/32) .. + 8; the three
  // products hi*hi, hi*lo, lo*hi accumulate in float32.
  static __device__ __forceinline__ void form_c(const Geo& g, const MergeLayout& ML, const _Float16* xh,
                                                const _Float16* xl, f16v acc[4]) {
    const int nb = ML.N / 32, ksteps = ML.K / 16;
    const size_t xs = (size_t)ML.K + 8;
    const int l = g.lane;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = g.wave + u * g.nw;
      f16v c = {};
      if (b < nb * nb) {
        const int J1 = b / nb, J2 = b - J1 * nb;
        const size_t ka = (size_t)(J1 * 32 + (l & 31)) * xs + 8 * (l >> 5);
        const size_t kb = (size_t)(J2 * 32 + (l & 31)) * xs + 8 * (l >> 5);
        for (int s = 0; s < ksteps; ++s) {
          const h8v a_h = *reinterpret_cast<const h8v*>(xh + ka + 16 * s);
          const h8v a_l = *reinterpret_cast<const h8v*>(xl + ka + 16 * s);
          const h8v b_h = *reinterpret_cast<const h8v*>(xh + kb + 16 * s);
          const h8v b_l = *reinterpret_cast<const h8v*>(xl + kb + 16 * s);
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_h, b_h, c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_h, b_l, c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_l, b_h, c, 0, 0, 0);
        }
      }
      acc[u] = c;
    }
  }

  // The blocks of form_c times 2^e, split, into C's area (row-major, N + 8
  // halves per row). Register r of lane l holds C[J1*32 + 8(r/4) + 4(l/32) + r%4][J2*32 + l%32];
  // C is symmetric, so each block is written to (J2, J1) with rows and columns
  // exchanged, four consecutive columns per store.
  static __device__ __forceinline__ void store_c(const Geo& g, const MergeLayout& ML, const f16v acc[4], int e,
                                                 _Float16* chh, _Float16* cll) {
    const int nb = ML.N / 32;
    const size_t cs = (size_t)ML.N + 8;
    const int l = g.lane;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = g.wave + u * g.nw;
      if (b < nb * nb) {
        const int J1 = b / nb, J2 = b - J1 * nb;
        const size_t row = (size_t)(J2 * 32 + (l & 31)) * cs;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          h4v hi, lo;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float x = ldexpf(acc[u][4 * r4 + t], e);
            const _Float16 h = (_Float16)x;
            hi[t] = h;
            lo[t] = (_Float16)__fsub_rn(x, (float)h);
          }
          const size_t col = (size_t)J1 * 32 + 8 * r4 + 4 * (l >> 5);
          *reinterpret_cast<h4v*>(chh + row + col) = hi;
          *reinterpret_cast<h4v*>(cll + row + col) = lo;
        }
      }
    }
  }

  // Y (N x pc) = C Q 2^qe in 16 x 16 output blocks over the wavefronts (each
  // wavefront's largest output magnitude to wmax[wave]):
  // C's split rows as the A operand, the basis times 2^qe split as B.
  // Lane l of a block reads C row M0 + l%16 and basis column n0 + l%16 at
  // 32 s + 8 (l/16) .. + 8 and gets Y[M0 + 4 (l/16) + r][n0 + l%16] back.
  static __device__ __forceinline__ void cq(const Geo& g, const MergeLayout& ML, const _Float16* chh,
                                            const _Float16* cll, const float* q, float* y, int qe, float* wmax) {
    const int N = ML.N;
    const int nbr = N / 16, nbc = ML.pc / 16;
    const size_t cs = (size_t)N + 8, bs = (size_t)N + 4;
    const int l = g.lane;
    float m = 0.f;
    for (int b = g.wave; b < nbr * nbc; b += g.nw) {
      const int M0 = (b % nbr) * 16, n0 = (b / nbr) * 16;
      const size_t ar = (size_t)(M0 + (l & 15)) * cs + 8 * (l >> 4);
      const float* qc = q + (size_t)(n0 + (l & 15)) * bs + 8 * (l >> 4);
      f4v acc = {};
      for (int s = 0; s < N / 32; ++s) {
        const h8v a_h = *reinterpret_cast<const h8v*>(chh + ar + 32 * s);
        const h8v a_l = *reinterpret_cast<const h8v*>(cll + ar + 32 * s);
        float v[8];
        loadf8(qc + 32 * s, v);
        h8v b_h, b_l;
        split8(v, qe, b_h, b_l);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_h, b_h, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_h, b_l, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_l, b_h, acc, 0, 0, 0);
      }
      *reinterpret_cast<f4v*>(y + (size_t)(n0 + (l & 15)) * bs + M0 + 4 * (l >> 4)) = acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(acc[r]));
    }
    m = wave_max(m);
    if (l == 0) wmax[g.wave] = m;
  }

  // a fixed pseudo-random sign for (row, column) (an integer hash's low bit)
  static __device__ __forceinline__ float pm1(int r, int c) {
    uint32_t h = (uint32_t)r * 0x9E3779B1u ^ (uint32_t)c * 0x85EBCA77u;
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    return (h & 1u) ? 1.f : -1.f;
  }

  // This wavefront's A fragments of C (creg layouts): its 16-row blocks
  // rb = wave + i * nw (i < 2), K steps s < N / 32 <= 4, high and low parts
  struct CFrag {
    h8v h[2][4], l[2][4];
  };

  static __device__ __forceinline__ void load_cfrag(const Geo& g, const MergeLayout& ML, const _Float16* chh,
                                                    const _Float16* cll, CFrag& F) {
    const int N = ML.N, nbr = N / 16;
    const size_t cs = (size_t)N + 8;
    const int l = g.lane;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rb = g.wave + i * g.nw;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (rb < nbr && s < N / 32) {
          const size_t at = (size_t)(rb * 16 + (l & 15)) * cs + 32 * s + 8 * (l >> 4);
          F.h[i][s] = *reinterpret_cast<const h8v*>(chh + at);
          F.l[i][s] = *reinterpret_cast<const h8v*>(cll + at);
        }
      }
    }
  }

  // cq with C's fragments in registers (creg: one 16-column block)
  static __device__ __forceinline__ void cq_reg(const Geo& g, const MergeLayout& ML, const CFrag& F, const float* q,
                                                float* y, int qe, float* wmax) {
    const int N = ML.N, nbr = N / 16;
    const size_t bs = (size_t)N + 4;
    const int l = g.lane;
    const float* qc = q + (size_t)(l & 15) * bs + 8 * (l >> 4);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rb = g.wave + i * g.nw;
      if (rb < nbr) {
        f4v acc = {};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (s < N / 32) {
            float v[8];
            loadf8(qc + 32 * s, v);
            h8v b_h, b_l;
            split8(v, qe, b_h, b_l);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(F.h[i][s], b_h, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(F.h[i][s], b_l, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(F.l[i][s], b_h, acc, 0, 0, 0);
          }
        }
        *reinterpret_cast<f4v*>(y + (size_t)(l & 15) * bs + rb * 16 + 4 * (l >> 4)) = acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(acc[r]));
      }
    }
    m = wave_max(m);
    if (l == 0) wmax[g.wave] = m;
  }

  // Largest magnitude over the lane's fragments of a basis (columns < p) and
  // its wavefront maximum
  template <int NC>
  static __device__ __forceinline__ float basis_max(const Geo& g, const float* src, int N, int p) {
    const size_t bs = (size_t)N + 4;
    float m = 0.f;
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      const int col = cb * 16 + (g.lane & 15);
      for (int s = 0; s < N / 32; ++s) {
        if (col < p) {
          float v[8];
          loadf8(src + (size_t)col * bs + 32 * s + 8 * (g.lane >> 4), v);
#pragma unroll
          for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(v[t]));
        }
      }
    }
    return wave_max(m);
  }

  // the lane's A/B fragment of basis column cb*16 + l%16 (zero past p), rows 32 s + 8 (l/16) .. + 8, split
  static __device__ __forceinline__ void basis_frag(const Geo& g, const float* src, int N, int p, int cb, int s,
                                                    int e, h8v& hi, h8v& lo) {
    const int col = cb * 16 + (g.lane & 15);
    float v[8];
    if (col < p) {
      loadf8(src + (size_t)col * ((size_t)N + 4) + 32 * s + 8 * (g.lane >> 4), v);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = 0.f;
    }
    split8(v, e, hi, lo);
  }

  // One CholeskyQR pass src -> dst (N x p bases, column-major, N + 4 floats
  // per column; dst's columns from p to pc become zero), to be followed by a
  // barrier of the caller. Wavefront 0 forms the p x p Gram matrix of src 2^e
  // on the matrix cores (split binary16, e from smax, a bound on src's magnitudes),
  // factors it (lane i holds row i; columns reach the other lanes by readlane)
  // and inverts the factor (lane c forms column c of L^-1, reading L's rows by
  // readlane); after a barrier
  // every thread applies dst = 2^e src L^-T to its rows. A column whose
  // remaining norm is below 1e-3 of its own (pivot below 1e-6 of its Gram
  // diagonal) gets a zero row in L^-1 and drops out. Returns, in every thread,
  // the ratio of the largest to the smallest live diagonal entry of L: an
  // estimate of src's condition number. P16 is p rounded up to 16, P8 is p
  // rounded up to a supported unrolled size.
  template <int P16, int P8>
  static __device__ __forceinline__ float orth_pass(const Geo& g, const MergeLayout& ML, const float* src, float* dst,
                                                    int p, float* ws, float* misc, float smax) {
    constexpr int NC = P16 / 16;
    const int N = ML.N;
    const size_t bs = (size_t)N + 4;
    const int l = g.lane;
    float* Lr = ws;                          // the Gram matrix
    float* Mi = ws + (kMaxCap + 1) * kWs;    // rows of L^-1
    if (g.wave == 0) {
      const int e = fit_exp(smax);
      // Gram blocks (a, b), a <= b: register r of lane l holds G[a*16 + 4(l/16) + r][b*16 + l%16]
      f4v G[NC][NC];
#pragma unroll
      for (int a0 = 0; a0 < NC; ++a0)
#pragma unroll
        for (int b0 = 0; b0 < NC; ++b0) G[a0][b0] = f4v{0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < N / 32; ++s) {
        h8v hi[NC], lo[NC];
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) basis_frag(g, src, N, p, cb, s, e, hi[cb], lo[cb]);
#pragma unroll
        for (int a0 = 0; a0 < NC; ++a0)
#pragma unroll
          for (int b0 = a0; b0 < NC; ++b0) {
            G[a0][b0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi[a0], hi[b0], G[a0][b0], 0, 0, 0);
            G[a0][b0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi[a0], lo[b0], G[a0][b0], 0, 0, 0);
            G[a0][b0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo[a0], hi[b0], G[a0][b0], 0, 0, 0);
          }
      }
      // to the scratch, row-major: every block exchanged (four consecutive
      // columns per store), the off-diagonal ones also as they are
#pragma unroll
      for (int a0 = 0; a0 < NC; ++a0)
#pragma unroll
        for (int b0 = a0; b0 < NC; ++b0) {
          *reinterpret_cast<f4v*>(Lr + (b0 * 16 + (l & 15)) * kWs + a0 * 16 + 4 * (l >> 4)) = G[a0][b0];
          if (a0 < b0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Lr[(a0 * 16 + 4 * (l >> 4) + r) * kWs + b0 * 16 + (l & 15)] = G[a0][b0][r];
          }
        }
      wave_sync_lds();
      // G = L L^T, lane i holding row i
      float row[P8];
      float dmine = 0.f;
      if constexpr (P8 <= 16) {
        // (unconditional reads: rows past 16 of the scratch hold nothing the
        // first 16 lanes use)
#pragma unroll
        for (int c = 0; c < P8; ++c) {
          const float v = Lr[l * kWs + c];
          row[c] = (l < p && c < p) ? v : 0.f;
        }
        const float gd = Lr[l * kWs + (l & 15)];
        const float gii = (l < p) ? gd : 0.f;
        chol16<P8, 0>(row, gii, dmine, l);
        float x[P8];
        linv16<P8, 0>(row, dmine, x, l, Mi, kWs);
      } else {
#pragma unroll
      for (int c = 0; c < P8; ++c) row[c] = (l < p && c < p) ? Lr[l * kWs + c] : 0.f;
      const float gii = (l < p) ? Lr[l * kWs + l] : 0.f;
#pragma unroll
      for (int k = 0; k < P8; ++k) {
        const float piv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row[k]), k));
        const float gkk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gii), k));
        const bool live = piv > 1e-6f * gkk && piv > 0.f;
        // 1/sqrt to about an ulp: the next pass (or CholeskyQR2) removes what this one leaves
        const float di = live ? __builtin_amdgcn_rsqf(piv) : 0.f;
        const float lik = __fmul_rn(row[k], di);
        row[k] = lik;
        if (l == k) dmine = di;
#pragma unroll
        for (int j = k + 1; j < P8; ++j) {
          const float ljk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lik), j));
          row[j] = __builtin_fmaf(-lik, ljk, row[j]);
        }
      }
      // L^-1: lane l forms column l, x_i = (i == l ? 1 : -sum_{t<i} L_it x_t) / L_ii
      // (zero above l), taking row i of L (lane i's `row`) and 1/L_ii by readlane
      if (true) {
        float x[P8];
#pragma unroll
        for (int i = 0; i < P8; ++i) {
          float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < i; ++t) {
            const float lit = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row[t]), i));
            s4[t & 3] = __builtin_fmaf(lit, x[t], s4[t & 3]);
          }
          const float su = __fadd_rn(__fadd_rn(s4[0], s4[1]), __fadd_rn(s4[2], s4[3]));
          const float di = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dmine), i));
          x[i] = (i == l) ? di : ((i < l) ? 0.f : -__fmul_rn(di, su));
          if (l < P8) Mi[i * kWs + l] = x[i];
        }
      }
      }
      // condition estimate: the live diagonal entries of L are the 1/dinv
      const bool lv = l < p && dmine > 0.f;
      const float dmx = wave_max(lv ? dmine : 0.f);
      const float dmn = -wave_max(lv ? -dmine : -INFINITY);
      if (l == 0) {
        misc[kMiscOrth] = (dmx > 0.f) ? dmx / dmn : 1.f;
        misc[kMiscOrth + 1] = __int_as_float(e);
      }
    }
    __syncthreads();
    const int e = __float_as_int(misc[kMiscOrth + 1]);
    const float kappa = misc[kMiscOrth];
    // dst = 2^e src L^-T: lane -> row, and a wavefront-uniform group of columns
    // (c = gm, gm + G, ...) per wavefront, so that no lane idles on another's columns
    const int nrg = (N + 63) / 64;           // row groups of 64
    const int G = g.nw / nrg;                // column groups
    const int gm = g.wave / nrg;
    const int r = (g.wave - gm * nrg) * 64 + l;
    uint32_t mine = 0;                       // this group's columns
    for (int c = gm; c < P8; c += G) mine |= 1u << c;
    if (gm < G && r < N) {
      float yv[P8];
#pragma unroll
      for (int c = 0; c < P8; ++c) yv[c] = (c < p) ? ldexpf(src[(size_t)c * bs + r], e) : 0.f;
#pragma unroll
      for (int c = 0; c < P8; ++c) {
        if (!((mine >> c) & 1u)) continue;   // wavefront-uniform
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t4 = 0; t4 <= c; t4 += 4) {
          const f4v M4 = *reinterpret_cast<const f4v*>(Mi + c * kWs + t4);
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (t4 + t <= c) s4[t] = __builtin_fmaf(M4[t], yv[t4 + t], s4[t]);
        }
        dst[(size_t)c * bs + r] = (c < p) ? __fadd_rn(__fadd_rn(s4[0], s4[1]), __fadd_rn(s4[2], s4[3])) : 0.f;
      }
      if (gm == 0)
        for (int c = P8; c < ML.pc; ++c) dst[(size_t)c * bs + r] = 0.f;
    }
    return kappa;
  }

  // H = Q^T Y (p x p, Y = C Q 2^kQScale) on the matrix cores in wavefront 0,
  // symmetrised into h (row stride kSm), with `hs` as scratch. Returns E with
  // H = 2^E Q^T C Q.
  template <int P16>
  static __device__ __forceinline__ int rr_matrix(const Geo& g, const MergeLayout& ML, const float* q, const float* y,
                                                  int p, float* h, float* hs) {
    constexpr int NC = P16 / 16;
    const int N = ML.N;
    const int l = g.lane;
    const int ey = fit_exp(basis_max<NC>(g, y, N, p));
    f4v H4[NC][NC];
#pragma unroll
    for (int a0 = 0; a0 < NC; ++a0)
#pragma unroll
      for (int b0 = 0; b0 < NC; ++b0) H4[a0][b0] = f4v{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < N / 32; ++s) {
      h8v qh[NC], ql[NC], yh[NC], yl[NC];
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) {
        basis_frag(g, q, N, p, cb, s, kQScale, qh[cb], ql[cb]);
        basis_frag(g, y, N, p, cb, s, ey, yh[cb], yl[cb]);
      }
#pragma unroll
      for (int a0 = 0; a0 < NC; ++a0)
#pragma unroll
        for (int b0 = 0; b0 < NC; ++b0) {
          H4[a0][b0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[a0], yh[b0], H4[a0][b0], 0, 0, 0);
          H4[a0][b0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[a0], yl[b0], H4[a0][b0], 0, 0, 0);
          H4[a0][b0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql[a0], yh[b0], H4[a0][b0], 0, 0, 0);
        }
    }
#pragma unroll
    for (int a0 = 0; a0 < NC; ++a0)
#pragma unroll
      for (int b0 = 0; b0 < NC; ++b0)
#pragma unroll
        for (int r = 0; r < 4; ++r) hs[(a0 * 16 + 4 * (l >> 4) + r) * kSm + b0 * 16 + (l & 15)] = H4[a0][b0][r];
    wave_sync_lds();
    for (int e = l; e < p * p; e += 64) {
      const int i = e / p, j = e - i * p;
      h[i * kSm + j] = 0.5f * (hs[i * kSm + j] + hs[j * kSm + i]);
    }
    return 2 * kQScale + ey;
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

  // cos and sin of the rotation that zeroes H_ab (a < b) given H_aa, H_bb, H_ab;
  // index a gets (J_aa, J_ba) = (c, -sn) and b gets (J_bb, J_ab) = (c, sn)
  // Branch-free: with d = H_bb - H_aa and e = 2 H_ab, the smaller root of
  // t^2 + 2 (d / e) t - 1 = 0 is t = sgn(d) e / (|d| + sqrt(d^2 + e^2)) (sgn by
  // d's sign bit), and e = 0 gives the identity. The angle to about an ulp:
  // the rotations stay orthogonal to that order. (|d|, |e| stay far below
  // 2^63: H is Q^T C Q scaled into binary16 range.)
  static __device__ __forceinline__ void rot_cs(float haa, float hbb, float hab, float& c, float& sn) {
    const float d = hbb - haa, e = 2.f * hab;
    const float r = __builtin_amdgcn_sqrtf(d * d + e * e);
    const float sd = (__float_as_int(d) < 0) ? -1.f : 1.f;   // the sign bit of d
    float t = (sd * e) * __builtin_amdgcn_rcpf(fabsf(d) + r);
    t = (e != 0.f) ? t : 0.f;
    c = __builtin_amdgcn_rsqf(t * t + 1.f);
    sn = t * c;
  }

  // Cyclic Jacobi on the symmetric p x p matrix at H (row stride kSm), all
  // threads, one barrier per round. Round r applies the P/2 disjoint rotations
  // of the round-robin schedule, whose coefficients and partners are in the
  // table `rcur`: each thread writes its elements of J^T H J and V J into the
  // other buffers, and the thread owning the element (a, b), a < b, that is a
  // pair of the next round also forms the new H_aa and H_bb and publishes the
  // next rotation of a and b (an index paired with the padding player gets the
  // identity from its diagonal element's thread). The sweep stops at its start
  // once the off-diagonal part's squared norm is below 1e-4 of the diagonal's
  // (eigenvector errors of 1e-2 change the rank-k error only in the second
  // order). On return H holds the eigenvalues on its diagonal and V the
  // eigenvectors in its columns.
  static __device__ __forceinline__ void jacobi(const Geo& g, int p, float*& H, float*& V, float*& Hn, float*& Vn,
                                                float* misc, float4* rot) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int P = (p + 1) & ~1;
    const int ne = p * p;
    float4* rcur = rot;
    float4* rnxt = rot + kMaxCap;
    float off = 0.f, dia = 0.f;
    // the elements e = tid, tid + nt, ... of the p x p matrices (one per thread
    // on the large blocks; the stride covers blocks of fewer threads)
    for (int e = tid; e < ne; e += nt) {
      const int i = e / p, j = e - (e / p) * p;
      V[i * kSm + j] = (i == j) ? 1.f : 0.f;
      const float h = H[i * kSm + j];
      if (i == j) dia = __builtin_fmaf(h, h, dia);
      else off = __builtin_fmaf(h, h, off);
      const int y = rr_partner(i, 0, P);
      if (i == j && y >= p) rcur[i] = make_float4(1.f, 0.f, __int_as_float(i), 0.f);
      if (i < j && y == j) {
        float c, sn;
        rot_cs(H[i * kSm + i], H[j * kSm + j], h, c, sn);
        rcur[i] = make_float4(c, -sn, __int_as_float(j), 0.f);
        rcur[j] = make_float4(c, sn, __int_as_float(i), 0.f);
      }
    }
    off = wave_sum(off);
    dia = wave_sum(dia);
    if (g.lane == 0) {
      misc[kMiscJac + 2 * g.wave] = off;
      misc[kMiscJac + 2 * g.wave + 1] = dia;
    }
    __syncthreads();
    int round = 0, sweep = 0;
    for (;;) {
      if (round == 0) {
        // the norms at the start of this sweep (double buffered by sweep parity)
        const float* pb = misc + kMiscJac + (sweep & 1) * 16;
        float so = 0.f, sd = 0.f;
        for (int w = 0; w < g.nw; ++w) {
          so += pb[2 * w];
          sd += pb[2 * w + 1];
        }
        if (!(so > 1e-4f * sd) || sweep == kJacobiSweeps) break;   // (a NaN matrix stops too)
      }
      const int nxt = (round + 1 == P - 1) ? 0 : round + 1;
      float off2 = 0.f, dia2 = 0.f;
      for (int e = tid; e < ne; e += nt) {
        const int i = e / p, j = e - (e / p) * p;
        const float4 ri = rcur[i], rj = rcur[j];
        const int pi = __float_as_int(ri.z), pj = __float_as_int(rj.z);
        const float hn = ri.x * (rj.x * H[i * kSm + j] + rj.y * H[i * kSm + pj]) +
                         ri.y * (rj.x * H[pi * kSm + j] + rj.y * H[pi * kSm + pj]);
        Hn[i * kSm + j] = hn;
        Vn[i * kSm + j] = rj.x * V[i * kSm + j] + rj.y * V[i * kSm + pj];
        if (nxt == 0) {
          if (i == j) dia2 = __builtin_fmaf(hn, hn, dia2);
          else off2 = __builtin_fmaf(hn, hn, off2);
        }
        const int y = rr_partner(i, nxt, P);
        if (i == j && y >= p) rnxt[i] = make_float4(1.f, 0.f, __int_as_float(i), 0.f);
        if (i < j && y == j) {
          // the pair's new diagonal entries, as their own threads form them
          const float hii = ri.x * (ri.x * H[i * kSm + i] + ri.y * H[i * kSm + pi]) +
                            ri.y * (ri.x * H[pi * kSm + i] + ri.y * H[pi * kSm + pi]);
          const float hjj = rj.x * (rj.x * H[j * kSm + j] + rj.y * H[j * kSm + pj]) +
                            rj.y * (rj.x * H[pj * kSm + j] + rj.y * H[pj * kSm + pj]);
          float c, sn;
          rot_cs(hii, hjj, hn, c, sn);
          rnxt[i] = make_float4(c, -sn, __int_as_float(j), 0.f);
          rnxt[j] = make_float4(c, sn, __int_as_float(i), 0.f);
        }
      }
      if (nxt == 0) {
        off2 = wave_sum(off2);
        dia2 = wave_sum(dia2);
        if (g.lane == 0) {
          float* pb = misc + kMiscJac + ((sweep + 1) & 1) * 16;
          pb[2 * g.wave] = off2;
          pb[2 * g.wave + 1] = dia2;
        }
      }
      __syncthreads();
      float* t = H; H = Hn; Hn = t;
      t = V; V = Vn; Vn = t;
      float4* tr = rcur; rcur = rnxt; rnxt = tr;
      round = nxt;
      if (round == 0) ++sweep;
    }
  }

  static __device__ __forceinline__ float bperm(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(lane << 2, __float_as_int(v)));
  }

  // Slot pairs and their rotation for the one-wavefront Jacobi: players of the
  // round-robin schedule (circle method: position 0 fixed, positions 1 .. 15
  // rotate by one per round, pairs (m, 15 - m)) sit in slots 2m (position m)
  // and 2m + 1 (position 15 - m), so the pairs are always the slot pairs of the
  // 2 x 2 blocks. From one round to the next, slot half (m, tau) (tau = 0 for
  // slot 2m, 1 for 2m + 1) takes the player of rowmap(m, tau).
  static __device__ __forceinline__ void rowmap(int m, int tau, int& m2, int& tau2) {
    if (tau == 0) {
      if (m == 0) { m2 = 0; tau2 = 0; }
      else if (m == 1) { m2 = 0; tau2 = 1; }
      else { m2 = m - 1; tau2 = 0; }
    } else {
      if (m < 7) { m2 = m + 1; tau2 = 1; }
      else { m2 = 7; tau2 = 0; }
    }
  }

  // Cyclic Jacobi on the symmetric p x p matrix at H (p <= 16, padded to 16
  // with zeros), in wavefront 0 alone and in registers: lane L holds the 2 x 2
  // blocks (L/8, L%8) of H and of V (V's rows are the basis index, its columns
  // the slots). A round rotates every slot pair (2m, 2m+1) by the angle its
  // diagonal block gives (the same rotation as the all-thread version's), then
  // moves rows and columns of H and columns of V to the next round's slots
  // through the scratch `hs`, `vs` ([64][4] floats each): one store of every
  // rotated block, then one batch of loads that brings each lane its new
  // blocks and the new diagonal blocks of its pairs, from which it forms both
  // of its next rotations itself. The sweep stops at its start once the
  // off-diagonal part's squared norm is below 1e-4 of the diagonal's. On
  // return H's diagonal holds the 16 slots' eigenvalues and V's columns their
  // eigenvectors (padding slots: eigenvalue 0, eigenvector on a padding row).
  static __device__ __forceinline__ void jacobi16(const Geo& g, int p, float* H, float* V, float* hs, float* vs) {
    const int l = g.lane;
    const int A = l >> 3, B = l & 7;
    const bool dg = A == B;
    float h[4], v[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int r = 2 * A + (d >> 1), c = 2 * B + (d & 1);
      h[d] = (r < p && c < p) ? H[r * kSm + c] : 0.f;
      v[d] = (r == c) ? 1.f : 0.f;
    }
    auto hp = [&](int r, int c) { return (r < p && c < p) ? H[r * kSm + c] : 0.f; };
    // this round's rotations of pairs A and B, from their diagonal blocks
    float cA, sA, cB, sB;
    rot_cs(hp(2 * A, 2 * A), hp(2 * A + 1, 2 * A + 1), hp(2 * A, 2 * A + 1), cA, sA);
    rot_cs(hp(2 * B, 2 * B), hp(2 * B + 1, 2 * B + 1), hp(2 * B, 2 * B + 1), cB, sB);
    // where each value comes from after a round (fixed): own block's four H
    // and four V values, and the new diagonal blocks (aa, bb, ab) of A and B
    int hsrc[4], vsrc[4], dA[3], dB[3];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      int ra, rt, cb, ct;
      rowmap(A, d >> 1, ra, rt);
      rowmap(B, d & 1, cb, ct);
      hsrc[d] = 4 * (8 * ra + cb) + 2 * rt + ct;
      vsrc[d] = 4 * (8 * A + cb) + 2 * (d >> 1) + ct;
    }
    {
      int r0, t0, r1, t1;
      rowmap(A, 0, r0, t0);
      rowmap(A, 1, r1, t1);
      dA[0] = 4 * (8 * r0 + r0) + 2 * t0 + t0;
      dA[1] = 4 * (8 * r1 + r1) + 2 * t1 + t1;
      dA[2] = 4 * (8 * r0 + r1) + 2 * t0 + t1;
      rowmap(B, 0, r0, t0);
      rowmap(B, 1, r1, t1);
      dB[0] = 4 * (8 * r0 + r0) + 2 * t0 + t0;
      dB[1] = 4 * (8 * r1 + r1) + 2 * t1 + t1;
      dB[2] = 4 * (8 * r0 + r1) + 2 * t0 + t1;
    }
    for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
      float off = dg ? __fmaf_rn(h[1], h[1], h[2] * h[2])
                     : __fmaf_rn(h[0], h[0], __fmaf_rn(h[1], h[1], __fmaf_rn(h[2], h[2], h[3] * h[3])));
      float dia = dg ? __fmaf_rn(h[0], h[0], h[3] * h[3]) : 0.f;
      off = wave_sum(off);
      dia = wave_sum(dia);
      if (!(off > 1e-4f * dia)) break;   // (a NaN matrix stops too)
      for (int round = 0; round < 15; ++round) {
        // J = [[c, s], [-s, c]]: T = H J_B, H' = J_A^T T, V' = V J_B
        const float t0 = h[0] * cB - h[1] * sB, t1 = h[0] * sB + h[1] * cB;
        const float t2 = h[2] * cB - h[3] * sB, t3 = h[2] * sB + h[3] * cB;
        f4v m, w;
        m[0] = cA * t0 - sA * t2;
        m[1] = cA * t1 - sA * t3;
        m[2] = sA * t0 + cA * t2;
        m[3] = sA * t1 + cA * t3;
        if (dg) {   // the rotation zeroes the pair's off-diagonal element
          m[1] = 0.f;
          m[2] = 0.f;
        }
        w[0] = v[0] * cB - v[1] * sB;
        w[1] = v[0] * sB + v[1] * cB;
        w[2] = v[2] * cB - v[3] * sB;
        w[3] = v[2] * sB + v[3] * cB;
        *reinterpret_cast<f4v*>(hs + 4 * l) = m;
        *reinterpret_cast<f4v*>(vs + 4 * l) = w;
        wave_sync_lds();
        // the next round's slots
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          h[d] = hs[hsrc[d]];
          v[d] = vs[vsrc[d]];
        }
        const float aa = hs[dA[0]], ab = hs[dA[2]], bA = hs[dA[1]];
        const float ba = hs[dB[0]], bb = hs[dB[1]], bab = hs[dB[2]];
        wave_sync_lds();   // every lane has read before the next round's stores
        rot_cs(aa, bA, ab, cA, sA);
        rot_cs(ba, bb, bab, cB, sB);
      }
    }
    // eigenvalues on the diagonal, eigenvectors in the columns (slot order)
    if (dg) {
      H[(2 * A) * kSm + 2 * A] = h[0];
      H[(2 * A + 1) * kSm + 2 * A + 1] = h[3];
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) V[(2 * A + (d >> 1)) * kSm + 2 * B + (d & 1)] = v[d];
  }

  // The rank-k factors of R (2^eR R split in X's area, R in registers),
  // written to the bypass's first k columns as U_k S^1/2 and V_k S^1/2.
  template <int P16, int P8>
  static __device__ __forceinline__ void factor(const StepArgs& a, const Geo& g, const MergeLayout& ML,
                                                const float R[8][8], float rmax, int p, int k, __half* U,
                                                __half* W) {
    extern __shared__ float lds[];
    const int tid = threadIdx.x, nt = blockDim.x;
    const int N = ML.N;
    const size_t bs = (size_t)N + 4;
    float* misc = lds + ML.misc;
    _Float16* lh = reinterpret_cast<_Float16*>(lds);
    const int eR = fit_exp(rmax);
    write_x(g, ML, R, eR, lh + ML.xh, lh + ML.xl);
    __syncthreads();
    f16v acc[4];
    form_c(g, ML, lh + ML.xh, lh + ML.xl, acc);
    __syncthreads();   // X's area becomes C's
    // C' = X^T X <= K 2^30 entrywise; 2^eC C' <= 2^14 fits binary16 with its low part
    const int eC = -(16 + (32 - __builtin_clz((unsigned)ML.K - 1u)));
    _Float16* chh = lh + ML.ch;
    _Float16* cll = lh + ML.cl;
    store_c(g, ML, acc, eC, chh, cll);
    CFrag cf;
    if (ML.creg) {
      // every wavefront takes its rows of C into registers; then C's area is free
      __syncthreads();
      load_cfrag(g, ML, chh, cll, cf);
      __syncthreads();
    }
    // the start basis: the bypass's factors on the narrow side, which span L's
    // row (or column) space; all of them are read before any is rewritten.
    // An all-zero column (the slot of an earlier merge's empty residual) would
    // leave the basis short of rank, so it gets a fixed pseudo-random +-1
    // pattern instead. The largest magnitude sets the first product's binary16
    // scale. Wavefront w takes columns w, w + nw, ... (N <= 128: two rows per lane).
    float* Qb = lds + ML.q;
    float* Yb = lds + ML.y;
    float* wsc = lds + ML.ws;
    const __half* F = ML.right ? W : U;
    float fm = 0.f;
    for (int c = g.wave; c < ML.pc; c += g.nw) {
      const int r0 = g.lane, r1 = g.lane + 64;
      float v0 = 0.f, v1 = 0.f;
      if (c < p) {
        if (r0 < N) v0 = __half2float(F[(size_t)c * N + r0]);
        if (r1 < N) v1 = __half2float(F[(size_t)c * N + r1]);
      }
      float cm = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
      if (c < p && !(cm > 0.f)) {
        v0 = pm1(r0, c);
        v1 = pm1(r1, c);
        cm = 1.f;
      }
      if (r0 < N) Qb[(size_t)c * bs + r0] = v0;
      if (r1 < N) Qb[(size_t)c * bs + r1] = v1;
      fm = fmaxf(fm, cm);
    }
    if (g.lane == 0) misc[kMiscWave + g.wave] = fm;
    __syncthreads();
    for (int w = 0; w < g.nw; ++w) fm = fmaxf(fm, misc[kMiscWave + w]);
    const int iters = (p >= 8 * k + 8) ? kMergeItersWide : (p >= 3 * k + 4) ? kMergeItersMid : kMergeItersNarrow;
    float kappa = 1.f;
    // (the non-finite flags' slots: read long before, many barriers back)
    float* wmax = misc + kMiscWave + 8;
    for (int it = 0; it < iters;) {
      if (ML.creg) cq_reg(g, ML, cf, Qb, Yb, it == 0 ? fit_exp(fm) : kQScale, wmax);
      else cq(g, ML, chh, cll, Qb, Yb, it == 0 ? fit_exp(fm) : kQScale, wmax);
      __syncthreads();
      ++it;
      // a well-conditioned basis takes a second product before it is
      // orthonormalised again (never the last one, so that the final basis
      // stays well conditioned): the condition number grows by at most the
      // product's, about the last estimate (uniform: every thread read it)
      if (it + 1 < iters && kappa <= kDoubleKappa) {
        float ym = 0.f;
        for (int w = 0; w < g.nw; ++w) ym = fmaxf(ym, wmax[w]);
        __syncthreads();   // the maxima are read before the next product rewrites them
        if (ML.creg) cq_reg(g, ML, cf, Yb, Qb, fit_exp(ym), wmax);
        else cq(g, ML, chh, cll, Yb, Qb, fit_exp(ym), wmax);
        __syncthreads();
        ++it;
        float* t = Qb;
        Qb = Yb;
        Yb = t;
      }
      // the product's largest magnitude (its wavefronts' maxima, out before the barrier)
      float ym = 0.f;
      for (int w = 0; w < g.nw; ++w) ym = fmaxf(ym, wmax[w]);
      kappa = orth_pass<P16, P8>(g, ML, Yb, Qb, p, wsc, misc, ym);
      __syncthreads();
    }
    // CholeskyQR's loss of orthogonality grows like the square of the
    // condition number times the Gram matrix's precision (about 2^-22 here):
    // below 20 it stays under 1e-4, which changes the rank-k error by far
    // less than its tolerance; above, a second pass (CholeskyQR2). Uniform:
    // every thread read the same estimate.
    if (!(kappa <= 20.f)) {
      orth_pass<P16, P8>(g, ML, Qb, Yb, p, wsc, misc, 1.f);   // unit columns: entries below 1
      __syncthreads();
      float* t = Qb;
      Qb = Yb;
      Yb = t;
    }
    // Rayleigh-Ritz on Q^T C Q
    if (ML.creg) cq_reg(g, ML, cf, Qb, Yb, kQScale, wmax);
    else cq(g, ML, chh, cll, Qb, Yb, kQScale, wmax);
    __syncthreads();
    float* H = lds + ML.h0;
    float* Hn = lds + ML.h1;
    float* V = lds + ML.v0;
    float* Vn = lds + ML.v1;
    if (g.wave == 0) {
      const int eh = rr_matrix<P16>(g, ML, Qb, Yb, p, H, Hn);
      // H = 2^(eh + eC + 2 eR) Q^T R^T R Q (or R R^T)
      if (g.lane == 0) misc[kMiscFlag + 1] = __int_as_float(eh + eC + 2 * eR);
    }
    __syncthreads();
    // p <= 16: the one-wavefront Jacobi, whose 16 slots are ranked below
    int pr = p;
    if constexpr (P16 == 16) {
      if (g.wave == 0) jacobi16(g, p, H, V, Hn, Vn);
      __syncthreads();
      pr = 16;
    } else {
      jacobi(g, p, H, V, Hn, Vn, misc, reinterpret_cast<float4*>(lds + ML.rot));
    }
    // order of the eigenvalues, largest first (ties by index)
    int* order = reinterpret_cast<int*>(misc + kMiscOrder);
    float* sroot = misc + kMiscSroot;
    float* sinv = misc + kMiscSinv;
    if (g.wave == 0 && g.lane < pr) {
      // a NaN eigenvalue sorts last, so the ranks stay a permutation
      auto key = [](float v) { return v == v ? v : -INFINITY; };
      const float lam = key(H[g.lane * kSm + g.lane]);
      int rank = 0;
      for (int j = 0; j < pr; ++j) {
        const float lj = key(H[j * kSm + j]);
        rank += (lj > lam || (lj == lam && j < g.lane)) ? 1 : 0;
      }
      order[rank] = g.lane;
    }
    __syncthreads();
    if (g.wave == 0 && g.lane < k) {
      const int etot = __float_as_int(misc[kMiscFlag + 1]);
      const float lam = ldexpf(H[order[g.lane] * kSm + order[g.lane]], -etot);   // sigma^2
      const float sr = lam > 0.f ? __fsqrt_rn(__fsqrt_rn(lam)) : 0.f;              // sigma^(1/2)
      sroot[g.lane] = sr;
      sinv[g.lane] = sr > 0.f ? 1.0f / sr : 0.f;
    }
    // the narrow side's singular vectors v_m = Q V[:, order[m]] feed the
    // product with R (C's area is free now)
    MergeLds S;
    S.zt = lds + ML.zt;
    S.yt = lds + ML.yt;
    S.part = lds + ML.part;
    const int zs = merge_zs(a.dv), ys = merge_ys(a.dk);
    float* nv = ML.right ? S.zt : S.yt;
    const int ns = ML.right ? zs : ys;
    for (int e = tid; e < k * N; e += nt) {
      const int m = e / N, r = e - m * N;
      const int oc = order[m];
      float u = 0.f;
      for (int c = 0; c < p; ++c) u = __builtin_fmaf(Qb[(size_t)c * bs + r], V[c * kSm + oc], u);
      nv[(size_t)m * ns + r] = u;
    }
    __syncthreads();
    // the other side: R v_m (d_k) or R^T v_m (d_v)
    if (ML.right) prod_rz(a, g, R, S, k);
    else prod_rty(a, g, R, S, k);
    // U column m: (R v_m) sigma^-1/2 (v_m on the right) or v_m sigma^1/2; W column m the other way round
    const float* uscale = ML.right ? sinv : sroot;
    const float* wscale = ML.right ? sroot : sinv;
    // sign of each U column: its largest-magnitude entry (first on ties) is positive
    float* sgn = misc + kMiscSign;
    for (int mcol = g.wave; mcol < k; mcol += g.nw) {
      float best = -1.f, bval = 0.f;
      int bidx = 0x7fffffff;
      for (int i = g.lane; i < a.dk; i += 64) {
        const float u = S.yt[(size_t)mcol * ys + i] * uscale[mcol];
        // judged on the value as stored (binary16, whose rounding is odd-symmetric)
        const float au = fabsf(__half2float(__float2half_rn(u)));
        if (au > best || (au == best && i < bidx)) {
          best = au;
          bval = u;
          bidx = i;
        }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ob = __shfl_xor(best, m, 64), ov = __shfl_xor(bval, m, 64);
        const int oi = __shfl_xor(bidx, m, 64);
        if (ob > best || (ob == best && oi < bidx)) {
          best = ob;
          bval = ov;
          bidx = oi;
        }
      }
      if (g.lane == 0) sgn[mcol] = (bval < 0.f) ? -1.f : 1.f;
    }
    __syncthreads();
    for (int e = tid; e < k * a.dk; e += nt) {
      const int m = e / a.dk, i = e - m * a.dk;
      U[(size_t)m * a.dk + i] = __float2half_rn(sgn[m] * (S.yt[(size_t)m * ys + i] * uscale[m]));
    }
    for (int e = tid; e < k * a.dv; e += nt) {
      const int m = e / a.dv, j = e - m * a.dv;
      W[(size_t)m * a.dv + j] = __float2half_rn(sgn[m] * (S.zt[(size_t)m * zs + j] * wscale[m]));
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
    const MergeLayout ML = merge_layout(a.dk, a.dv, g.wrw, g.wcw, a.cap, a.lrb_k, a.merge_chunk);
    float* misc = lds + ML.misc;

    uint32_t flags = 0;
    // the bypass factors go through LDS; L is formed once from them and kept for R
    __half* us = reinterpret_cast<__half*>(lds);
    __half* wst = us + (size_t)a.n * a.dk;
    uint32_t mk[8];
    float R[8][8];   // L, kept through the requantization
    switch (he.bits) {
      case 4: requantize<4>(a, he, tb, g, us, wst, mk, R, flags); break;
      case 6: requantize<6>(a, he, tb, g, us, wst, mk, R, flags); break;
      default: requantize<8>(a, he, tb, g, us, wst, mk, R, flags); break;
    }
    // the residual R = L on the elements that stayed in the bypass, its
    // largest magnitude and whether it is finite
    float am = 0.f;
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((mk[i] >> j) & 0x101u) R[i][j] = 0.f;
        const float v = fabsf(R[i][j]);
        bad = bad || !(v <= 3.4e38f);
        am = fmaxf(am, v);
      }
    am = wave_max(am);
    const bool wbad = any_lane(bad);
    if (g.lane == 0) {
      misc[kMiscWave + g.wave] = am;
      misc[kMiscWave + 8 + g.wave] = wbad ? 1.f : 0.f;
    }
    __syncthreads();   // the staging area is free; the maxima are out
    float rmax = 0.f;
    bool rbad = false;
    for (int w = 0; w < g.nw; ++w) {
      rmax = fmaxf(rmax, misc[kMiscWave + w]);
      rbad = rbad || misc[kMiscWave + 8 + w] != 0.f;
    }
    if (rbad) flags |= kStatusNonfinite;

    const int p = a.n;
    const int k = min(a.lrb_k, p);
    __half* U = reinterpret_cast<__half*>(tb + he.bypass_u);
    __half* W = reinterpret_cast<__half*>(tb + he.bypass_w);
    // a zero residual keeps zero factors; a non-finite one is flagged and dropped
    const int kf = (rmax > 0.f && !rbad) ? k : 0;
    // up to 8 kept columns the subspace iteration starts from at most 16 of
    // the bypass's columns (the first ones: the previous merge's factors
    // first), which keeps its small matrices to one wavefront
    const int pb = (k <= 8 && p > 16) ? 16 : p;
    if (kf > 0) {
      if (pb <= 8) factor<16, 8>(a, g, ML, R, rmax, pb, k, U, W);
      else if (pb <= 16) factor<16, 16>(a, g, ML, R, rmax, pb, k, U, W);
      else if (pb <= 20) factor<32, 20>(a, g, ML, R, rmax, pb, k, U, W);
      else if (pb <= 24) factor<32, 24>(a, g, ML, R, rmax, pb, k, U, W);
      else factor<32, 32>(a, g, ML, R, rmax, pb, k, U, W);
    }
    // the columns past the kept factors are empty
    for (int e = threadIdx.x; e < (a.cap - kf) * a.dk; e += blockDim.x)
      U[(size_t)kf * a.dk + e] = __float2half_rn(0.f);
    for (int e = threadIdx.x; e < (a.cap - kf) * a.dv; e += blockDim.x)
      W[(size_t)kf * a.dv + e] = __float2half_rn(0.f);

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
