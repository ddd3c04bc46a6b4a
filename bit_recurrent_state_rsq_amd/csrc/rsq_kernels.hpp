// Kernel arguments and the pieces shared by the decode, readout and merge
// kernels; host-side entry points to pick a kernel instance.
#pragma once
#include "rsq_device.hpp"

namespace rsq {

enum { kRetNet = 0, kMamba2 = 1, kGLA = 2, kGDN = 3 };
enum { kScaleDynamic = 0, kScalePersistent = 1, kScaleYoked = 2 };
// Compile-time feature variants of the decode kernel.
enum { kFeatPlain = 0, kFeatBdr = 1, kFeatBypass = 2, kFeatYoked = 3, kFeatF32 = 4, kFeatDiag = 5, kFeatHad = 6,
       kFeatPW = 7 };

struct StepArgs {
  uint8_t* tiles;            // state buffer + tiles offset
  const HeadEntry* heads;    // head table (device)
  uint32_t* status;          // device status word
  int64_t* hdr_t;            // header step count
  int32_t* hdr_n;            // header bypass fill
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  float* o;
  uint64_t batch_stride;
  int32_t H, dk, dv, group;
  int32_t smode;
  float trigger;
  int32_t bdr;
  float bdr_eps;
  int32_t bypass;            // 1 when a low-rank bypass is configured
  int32_t n;                 // bypass columns in use before this call
  int32_t cap;               // k + m
  int32_t lrb_k;
  float lrb_eps;
  int32_t in_bf16;           // q, k, v are bf16 (else fp32)
  int32_t scale_f16;         // step sizes are stored as fp16 (else fp32)
  int32_t hadamard;          // groups are stored rotated by the Sylvester-Hadamard matrix
  int32_t pw;                // pure-write window size W (0 = none); a.n = pairs held before the step
  int64_t t_next;
  // error accounting (kFeatDiag only): per tile 6 planes of d_k*d_v floats in
  // the fp32 chunk layout, optional |b|/step per element, 4 counters
  float* dg_acc;
  float* dg_ratio;
  uint32_t* dg_counts;
  // every head alike (same width; RetNet: same gamma): the head table entry
  // is `uni` with head_offset = h * uni_stride, so the kernels skip its load
  int32_t uniform;
  uint64_t uni_stride;
  HeadEntry uni;
  // bypass merge: columns per pass of its closing products with R
  int32_t merge_chunk;
  // decode steps of quantized states stage each wavefront's code chunks in
  // LDS (512 bytes per code bit and wavefront) from this byte offset on
  int32_t lds_stage;
};

// Head table entry of head h.
__device__ __forceinline__ HeadEntry head_entry(const StepArgs& a, int h) {
  if (a.uniform) {
    HeadEntry e = a.uni;
    e.head_offset = (uint64_t)h * a.uni_stride;
    return e;
  }
  return a.heads[h];
}

typedef void (*DecodeFn)(StepArgs);
DecodeFn decode_kernel_for(int model, int cl, int feat, int spec);
// the raised-priority twin of a decode kernel for grids resident at once, or nullptr
DecodeFn decode_boost_twin(DecodeFn fn);
DecodeFn readout_kernel_for(int cl);
DecodeFn merge_kernel_for(int cl);
// dynamic LDS (floats) of the merge kernel for a tile of d_k x d_v split into
// wrw x wcw wavefronts with `cap` bypass columns of which k are kept,
// reducing its closing products over `chunk` columns per pass
size_t merge_lds_floats(int dk, int dv, int wrw, int wcw, int cap, int k, int chunk);

// Decay of key row i of a tile (Table 1, A_t column).
__device__ __forceinline__ float row_decay(const StepArgs& a, const HeadEntry& he, int model,
                                           int tile, int i) {
  if (model == kRetNet) return he.gamma;
  if (model == kGLA) return a.alpha[(size_t)tile * a.dk + i];
  return a.alpha[tile];
}

__device__ __forceinline__ float in_elem(bool bf16, const void* p, size_t idx) {
  if (bf16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[idx]);
  return reinterpret_cast<const float*>(p)[idx];
}

// Sum over the 64 lanes of a wavefront in a fixed order (every lane gets it):
// lane pairs 1, 2, 4, 8, 16 apart by DPP / swizzle, then the two halves.
__device__ __forceinline__ float wave_sum64(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x201F));
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
}

// Bypass side of a decode step (Low-Rank Bypass of "Preserving Updates in
// Low-Bit Recurrent State Quantization"; all of B_t goes to the bypass):
//   U[:, c] <- RN16(a_i U_ic) for c < n, U[:, n] = fp16(k), W[:, n] = fp16(w),
// and z_c = sum_i U_ic q_i (c <= n) for the readout term W z, left in lds_z.
// Column c belongs to wavefront c mod nw, whose lanes stride over the rows:
// the loads of a column are coalesced, and each column's sum is one wave
// reduction (the readout that uses it is order-free).
__device__ __forceinline__ void bypass_decode_phase(const StepArgs& a, const HeadEntry& he, uint8_t* tb, int tile,
                                                    float* lds_z, int model) {
  __half* U = reinterpret_cast<__half*>(tb + he.bypass_u);
  __half* W = reinterpret_cast<__half*>(tb + he.bypass_w);
  const int n = a.n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  for (int c = wave; c <= n; c += nw) {
    __half* uc = U + (size_t)c * a.dk;
    float acc = 0.f;
    // four rows per lane at a time, all loads issued before the stores (which
    // could alias later loads for all the compiler knows)
    for (int i0 = lane; i0 < a.dk; i0 += 256) {
      float qv[4], av[4];
      __half uv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 64 * r;
        const bool ok = i < a.dk;
        qv[r] = ok ? in_elem(a.in_bf16, a.q, (size_t)tile * a.dk + i) : 0.f;
        if (c < n) {
          av[r] = ok ? row_decay(a, he, model, tile, i) : 0.f;
          uv[r] = ok ? uc[i] : __float2half_rn(0.f);
        } else {
          av[r] = ok ? in_elem(a.in_bf16, a.k, (size_t)tile * a.dk + i) : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 64 * r;
        if (i < a.dk) {
          const __half un = c < n ? mul_rn_half(av[r], uv[r]) : __float2half_rn(av[r]);
          uc[i] = un;
          acc = __builtin_fmaf(__half2float(un), qv[r], acc);
        }
      }
    }
    acc = wave_sum64(acc);
    if (lane == 0) lds_z[c] = acc;
  }
  // the delta rule's column is fp16(w), written by the step once w is known
  if (model != kGDN)
    for (int j = threadIdx.x; j < a.dv; j += blockDim.x)
      W[(size_t)n * a.dv + j] = __float2half_rn(in_elem(a.in_bf16, a.v, (size_t)tile * a.dv + j));
  __syncthreads();
}

// Gated DeltaNet with a bypass: the retrieval reads S = s_hat + U W^T, so it
// needs b = W (U^T k) with U and W as they were before this step:
//   z_c = pairwise sum over rows (row order) of fl(U_ic k_i)   -> zk[c]
//   b_j = fma chain over c = 0 .. n-1 of (W_jc, z_c), from 0   -> bz[j]
// This is the general form, for tiles the register path below does not hold:
// column c belongs to wavefront c mod nw, lane l takes rows l R .. l R + R - 1
// (R = d_k / 64, or one row for d_k < 64; d_k is a power of two), sums them
// pairwise and the lanes then meet 1, 2, 4, ..., 32 apart (wave_sum64), which
// is the pairwise tree over all rows. Ends with a barrier.
__device__ __forceinline__ void gdn_bypass_retrieval_loop(const StepArgs& a, const HeadEntry& he, const uint8_t* tb,
                                                          int tile, float* zk, float* bz) {
  const __half* U = reinterpret_cast<const __half*>(tb + he.bypass_u);
  const __half* W = reinterpret_cast<const __half*>(tb + he.bypass_w);
  const int n = a.n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int R = a.dk >= 64 ? a.dk >> 6 : 1;   // 1 .. 16
  for (int c = wave; c < n; c += nw) {
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = lane * R + r;
      p[r] = (r < R && i < a.dk)
                 ? __fmul_rn(__half2float(U[(size_t)c * a.dk + i]), in_elem(a.in_bf16, a.k, (size_t)tile * a.dk + i))
                 : 0.f;
    }
    // pairwise over the lane's rows: the entries past R are zero subtrees
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
      for (int r = 0; r < 16; r += 2 * h) p[r] = __fadd_rn(p[r], p[r + h]);
    const float z = wave_sum64(p[0]);
    if (lane == 0) zk[c] = z;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < a.dv; j += blockDim.x) {
    float b = 0.f;
    for (int c = 0; c < n; ++c) b = __builtin_fmaf(__half2float(W[(size_t)c * a.dv + j]), zk[c], b);
    bz[j] = b;
  }
  __syncthreads();
}

// The same bypass step with every load issued at kernel start, next to the
// state's own, and held in registers until the state's step is done. The
// loop above waits on a round trip per column, and on gfx9 a wait for a
// load also waits for every store issued before it, so there each column
// costs a load and a store round trip. Here the decay, the stores and the
// sums run after the state's step, with nothing left to wait for.
// Holds for d_k <= 256 (four rows per lane), at most kBypCols columns per
// wavefront and, for the readout term, at most kBypWCols columns per
// partial-sum thread group (P = blockDim / d_v groups).
constexpr int kBypCols = 4, kBypWCols = 8;
// the delta rule's path reads every W column of its thread's row j (the
// retrieval's b_j runs over all of them in order): columns 0 .. n - 1, n <
// kBypWColsGdn, go straight from memory to LDS at kernel start
constexpr int kBypWColsGdn = 16;
// LDS bytes of that staging area: whole 1 KB wavefront loads
__host__ __device__ inline int gdn_wstage_bytes(int dv) { return (kBypWColsGdn * dv * 2 + 1023) / 1024 * 1024; }
// ... and of U's columns 0 .. n - 1, each in a slot of whole 256-byte
// wavefront loads (one dword per lane), loaded by the wavefront that reads it
__host__ __device__ inline int gdn_ustage_slot(int dk) { return (dk * 2 + 255) / 256 * 256; }
__host__ __device__ inline int gdn_ustage_bytes(int dk) { return kBypWColsGdn * gdn_ustage_slot(dk); }
typedef __attribute__((address_space(1))) const void g_cvoid;
typedef __attribute__((address_space(3))) void l_void;
struct BypassRegs {
  // raw loaded bits: nothing is converted until bypass_store, after the
  // state's own loads have been issued. Lane l holds rows 4l .. 4l + 3.
  uint32_t qb[4];              // q_i (bf16 pairs in qb[0..1], or 4 fp32)
  float av[4];                 // a_i
  uint32_t kb[4];              // k_i (used by the wavefront that writes column n)
  uint32_t uv[kBypCols][2];    // U_ic of the wavefront's columns (binary16 pairs)
  // W_jc of this thread's readout columns (binary16 bits; the delta rule's
  // are in LDS)
  uint32_t wv[kBypWCols];
  uint32_t vb;                 // v_j (column n of W is fp16(v_j); not for the delta rule)
};

__device__ __forceinline__ bool bypass_regs_fit(const StepArgs& a, int model) {
  const int nw = blockDim.x >> 6, P = (int)(blockDim.x / a.dv);
  if (model == kGDN) return a.dk <= 256 && a.n + 1 <= kBypCols * nw && P >= 1 && a.n < kBypWColsGdn;
  return a.dk <= 256 && a.n + 1 <= kBypCols * nw && P >= 1 && a.n + 1 <= kBypWCols * P;
}

__device__ __forceinline__ uint32_t in_bits(bool bf16, const void* p, size_t idx) {
  if (bf16) return reinterpret_cast<const uint16_t*>(p)[idx];
  return reinterpret_cast<const uint32_t*>(p)[idx];
}
__device__ __forceinline__ float bits_in(bool bf16, uint32_t b) { return __uint_as_float(bf16 ? b << 16 : b); }
// four consecutive inputs from element idx (a multiple of 4): bf16 as two
// words in w[0..1], fp32 as four
__device__ __forceinline__ void in4_bits(bool bf16, const void* p, size_t idx, uint32_t w[4]) {
  if (bf16) {
    const uint2 t = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p) + idx);
    w[0] = t.x, w[1] = t.y, w[2] = 0u, w[3] = 0u;
  } else {
    const uint4 t = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint32_t*>(p) + idx);
    w[0] = t.x, w[1] = t.y, w[2] = t.z, w[3] = t.w;
  }
}
__device__ __forceinline__ float in4_at(bool bf16, const uint32_t w[4], int r) {
  if (bf16) return __uint_as_float((r & 1) ? (w[r >> 1] & 0xFFFF0000u) : (w[r >> 1] << 16));
  return __uint_as_float(w[r]);
}
// pins a loaded value to this point of the program: the conversions that
// follow stay here instead of being hoisted next to the load (which would
// make the load's wait come early)
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// Every load is unconditional, at an index clamped into the tile's sections
// (values past n or d_k are loaded and dropped): no branch separates the
// loads, so they all leave before the first wait. Four consecutive rows per
// lane make each column one 8-byte load.
__device__ __forceinline__ void bypass_load(const StepArgs& a, const HeadEntry& he, const uint8_t* tb, int tile,
                                            int model, bool bf16, BypassRegs& br, __half* wst, uint8_t* ust) {
  const uint16_t* U = reinterpret_cast<const uint16_t*>(tb + he.bypass_u);
  const uint16_t* W = reinterpret_cast<const uint16_t*>(tb + he.bypass_w);
  // column indices clamp to the last column the step uses (U: n - 1, W: n),
  // so the loads past it hit lines already fetched instead of new ones
  const int ulast = max(a.n - 1, 0), wlast = a.n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int i4 = min(4 * lane, a.dk - 4);
  in4_bits(bf16, a.q, (size_t)tile * a.dk + i4, br.qb);
  in4_bits(bf16, a.k, (size_t)tile * a.dk + i4, br.kb);
  if (model == kGLA) {
    const float4 t = *reinterpret_cast<const float4*>(a.alpha + (size_t)tile * a.dk + i4);
    br.av[0] = t.x, br.av[1] = t.y, br.av[2] = t.z, br.av[3] = t.w;
  } else {
    const float d = row_decay(a, he, model, tile, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) br.av[r] = d;
  }
  if (model == kGDN) {
    // U's columns c = wave + nw m < n into their LDS slots at ust + c slot:
    // one dword per lane per 256 bytes, a lane past the column reading the
    // column's last dword (into its slot's padding)
    const uint8_t* Ub = reinterpret_cast<const uint8_t*>(U);
    const int cb = a.dk * 2, slot = gdn_ustage_slot(a.dk);
#pragma unroll
    for (int m = 0; m < kBypCols; ++m) {
      const int c = wave + nw * m;
      if (c < a.n) {
        for (int t0 = 0; t0 < cb; t0 += 256) {
          const int off = min(t0 + 4 * lane, cb - 4);
          __builtin_amdgcn_global_load_lds((g_cvoid*)(Ub + (size_t)c * cb + off), (l_void*)(ust + (size_t)c * slot + t0), 4, 0, 0);
        }
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < kBypCols; ++m) {
      const int c = min(wave + nw * m, ulast);
      const uint2 t = *reinterpret_cast<const uint2*>(U + (size_t)c * a.dk + i4);
      br.uv[m][0] = t.x, br.uv[m][1] = t.y;
    }
  }
  // readout term: thread (pp, j) takes columns pp, pp + P, ... (column n is
  // fp16(v_j), written this step: taken from v, not read back). The delta
  // rule's thread holds all of row j's columns before n (its column n is
  // fp16(w_j), known only after the retrieval).
  const int P = (int)(blockDim.x / a.dv);
  const int j = threadIdx.x % a.dv, pp = threadIdx.x / a.dv;
  if (model == kGDN) {
    // W's columns 0 .. n - 1 (column-major, contiguous) into LDS at wst: one
    // 1 KB direct load per wavefront instruction, 16 bytes per lane at
    // wst + 1024 c + 16 lane; a lane past W's section reads its last 16
    // bytes instead (staged past the columns the step reads)
    const uint8_t* Wb = reinterpret_cast<const uint8_t*>(W);
    const int wbytes = a.n * a.dv * 2, wcap = a.cap * a.dv * 2;
    for (int c0 = 1024 * wave; c0 < wbytes; c0 += 1024 * nw) {
      const int off = min(c0 + 16 * lane, wcap - 16);
      __builtin_amdgcn_global_load_lds((g_cvoid*)(Wb + off), (l_void*)(reinterpret_cast<uint8_t*>(wst) + c0), 16, 0, 0);
    }
    (void)P;
    (void)pp;
    br.vb = 0u;
    return;
  }
#pragma unroll
  for (int m = 0; m < kBypWCols; ++m) br.wv[m] = W[(size_t)min(pp + P * m, wlast) * a.dv + j];
  br.vb = in_bits(bf16, a.v, (size_t)tile * a.dv + j);
}

// The delta rule's bypass retrieval from the register path (same sums and
// order as gdn_bypass_retrieval_loop): lane l holds rows 4l .. 4l + 3, so the
// lane's rows pairwise and then wave_sum64 give the pairwise row tree. Runs
// before the retrieval of the stored state; ends with a barrier.
__device__ __forceinline__ void gdn_bypass_retrieval_regs(const StepArgs& a, bool bf16, const BypassRegs& br,
                                                          float* zk, float* bz, const __half* wst, const uint8_t* ust) {
  const int n = a.n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const bool rows_ok = 4 * lane < a.dk;
  const int slot = gdn_ustage_slot(a.dk);
  // this wavefront's U columns, staged by itself, have landed
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int m = 0; m < kBypCols; ++m) {
    const int c = wave + nw * m;
    if (c >= n) break;
    const uint2 uw = *reinterpret_cast<const uint2*>(ust + (size_t)c * slot + 8 * min(lane, a.dk / 4 - 1));
    const uint32_t uu[2] = {uw.x, uw.y};
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const __half u = __ushort_as_half((uint16_t)(uu[r >> 1] >> (16 * (r & 1))));
      p[r] = __fmul_rn(__half2float(u), in4_at(bf16, br.kb, r));
    }
    const float acc = __fadd_rn(__fadd_rn(p[0], p[1]), __fadd_rn(p[2], p[3]));
    const float z = wave_sum64(rows_ok ? acc : 0.f);
    if (lane == 0) zk[c] = z;
  }
  // this wavefront's W staging loads have landed in LDS; after the barrier
  // every wavefront's have
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int P = (int)(blockDim.x / a.dv);
  const int j = threadIdx.x % a.dv, pp = threadIdx.x / a.dv;
  if (pp == 0) {
    float b = 0.f;
#pragma unroll
    for (int m = 0; m < kBypWColsGdn; ++m)
      if (m < n) b = __builtin_fmaf(__half2float(wst[(size_t)m * a.dv + j]), zk[m], b);
    bz[j] = b;
  }
  (void)P;
  __syncthreads();
}

// Decay and store of U, the new columns of U and W, and z_c = sum_i U_ic q_i
// in lds_z (the lane's four rows in order, then a wave reduction).
__device__ __forceinline__ void bypass_store(const StepArgs& a, const HeadEntry& he, uint8_t* tb, int tile,
                                             int model, bool bf16, BypassRegs& br, float* lds_z, const uint8_t* ust) {
  uint16_t* U = reinterpret_cast<uint16_t*>(tb + he.bypass_u);
  __half* W = reinterpret_cast<__half*>(tb + he.bypass_w);
  const int n = a.n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const bool rows_ok = 4 * lane < a.dk;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pin(br.qb[r]);
    pin(br.av[r]);
    pin(br.kb[r]);
  }
#pragma unroll
  for (int m = 0; m < kBypCols; ++m) {
    const int c = wave + nw * m;
    if (c > n) break;
    uint32_t uu[2];
    if (model == kGDN) {
      // (the wavefront's own staged column; column n is written, not read)
      const uint2 uw = c < n ? *reinterpret_cast<const uint2*>(ust + (size_t)c * gdn_ustage_slot(a.dk) + 8 * min(lane, a.dk / 4 - 1))
                             : make_uint2(0u, 0u);
      uu[0] = uw.x, uu[1] = uw.y;
    } else {
      pin(br.uv[m][0]);
      pin(br.uv[m][1]);
      uu[0] = br.uv[m][0], uu[1] = br.uv[m][1];
    }
    float acc = 0.f;
    uint16_t un[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const __half u = __ushort_as_half((uint16_t)(uu[r >> 1] >> (16 * (r & 1))));
      const __half h = c < n ? mul_rn_half(br.av[r], u) : __float2half_rn(in4_at(bf16, br.kb, r));
      un[r] = __half_as_ushort(h);
      acc = __builtin_fmaf(__half2float(h), in4_at(bf16, br.qb, r), acc);
    }
    if (rows_ok)
      *reinterpret_cast<uint2*>(U + (size_t)c * a.dk + 4 * lane) =
          make_uint2((uint32_t)un[0] | ((uint32_t)un[1] << 16), (uint32_t)un[2] | ((uint32_t)un[3] << 16));
    acc = wave_sum64(rows_ok ? acc : 0.f);
    if (lane == 0) lds_z[c] = acc;
  }
  const int P = (int)(blockDim.x / a.dv);
  const int j = threadIdx.x % a.dv, pp = threadIdx.x / a.dv;
  pin(br.vb);
  // column n of row j (the delta rule's, fp16(w_j), is written by the step)
  if (model != kGDN && pp == n % P) W[(size_t)n * a.dv + j] = __float2half_rn(bits_in(bf16, br.vb));
}

// Readout term of the register path: this thread's share of (W z)_j. The
// delta rule passes its new column's fp16(w_j) as w_new.
__device__ __forceinline__ float bypass_wz_part(const StepArgs& a, int model, bool bf16, BypassRegs& br,
                                                const float* lds_z, float w_new, const __half* wst) {
  const int P = (int)(blockDim.x / a.dv);
  const int pp = threadIdx.x / a.dv;
  const int cnt = a.n + 1;
  float part = 0.f;
  if (model == kGDN) {
    // thread pp takes columns pp, pp + P, ... of its held row
#pragma unroll
    for (int m = 0; m < kBypWColsGdn; ++m) {
      if (m < cnt && m % P == pp) {
        const __half wh = m == a.n ? __float2half_rn(w_new) : wst[(size_t)m * a.dv + (threadIdx.x % a.dv)];
        part = __builtin_fmaf(__half2float(wh), lds_z[m], part);
      }
    }
    return part;
  }
#pragma unroll
  for (int m = 0; m < kBypWCols; ++m) {
    const int c = pp + P * m;
    pin(br.wv[m]);
    const __half wh = c == a.n ? __float2half_rn(bits_in(bf16, br.vb)) : __ushort_as_half((uint16_t)br.wv[m]);
    if (c < cnt) part = __builtin_fmaf(__half2float(wh), lds_z[c], part);
  }
  return part;
}

}  // namespace rsq
