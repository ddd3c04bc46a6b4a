/*
 * rsq.h - C ABI of the fused low-bit recurrent-state decode step (gfx950).
 *
 * One decode step of a linear-attention / state-space recurrence whose
 * per-head state S (d_k x d_v) is stored as group-wise low-bit codes:
 *
 *   S_t = A_t S_{t-1} + B_t                       (Table 1 of "Preserving
 *                                                  Updates in Low-Bit Recurrent
 *                                                  State Quantization")
 *     RetNet  A = gamma I            B = k v^T
 *     Mamba2  A = alpha_t I          B = k v^T
 *     GLA     A = Diag(alpha_t)      B = k v^T
 *     GDN     A = alpha_t I          B = beta_t k (v - (A S_{t-1})^T k)^T
 *   o_t = S_t^T q_t    (read before requantization)
 *
 * after which the state is requantized (the abstract of the same page: a
 * recurrent state is requantized after every update) with dynamic,
 * persistent or reference-yoked step sizes (abstract of "When Dynamic
 * Scaling Fails: A Scale-State Feedback Governs Recurrent-State Quantization
 * in Linear-Attention and SSM LLMs"), optional Bounded Directional Rounding
 * and an optional Low-Rank Bypass merged every m steps ("Preserving Updates
 * ...", abstract, Fig. 3, Fig. 4, Table 6).
 *
 * Conventions for every call
 *  - Plain C, no exceptions cross the ABI. Every call returns rsq_status
 *    (RSQ_OK = 0, errors < 0) except rsq_last_error / rsq_abi_version.
 *  - "device" pointers are HIP device memory of the current device; "host"
 *    pointers are ordinary host memory. The caller owns all memory; the
 *    library allocates only the small host handle rsq_state.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call is
 *    stream-ordered and asynchronous except rsq_get_status and
 *    rsq_state_alloc(RSQ_ATTACH), which synchronize the stream.
 *  - Argument errors are detected on the host before anything is launched;
 *    the call then returns RSQ_E_* and rsq_last_error() describes it.
 *  - Calls on one state must not overlap in time on different streams.
 */
#ifndef RSQ_H
#define RSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RSQ_ABI_VERSION 3

typedef int32_t rsq_status;
enum {
  RSQ_OK = 0,
  RSQ_E_INVALID = -1,      /* bad argument or configuration */
  RSQ_E_UNSUPPORTED = -2,  /* valid, but a shape/feature this build does not run */
  RSQ_E_BUFFER = -3,       /* device buffer too small */
  RSQ_E_BYPASS_FULL = -4,  /* decode step with k+m bypass columns in use: merge first */
  RSQ_E_NO_BYPASS = -5,    /* merge on a state without a bypass */
  RSQ_E_HIP = -6,          /* a HIP runtime call failed */
  RSQ_E_ATTACH = -7        /* RSQ_ATTACH found a header that does not match the config */
};

/* Table 1 rows. */
enum { RSQ_RETNET = 0, RSQ_MAMBA2 = 1, RSQ_GLA = 2, RSQ_GDN = 3 };
/* Scale policies (abstract of "When Dynamic Scaling Fails ..."). */
enum { RSQ_SCALE_DYNAMIC = 0, RSQ_SCALE_PERSISTENT = 1, RSQ_SCALE_YOKED = 2 };
/* Element types. */
enum { RSQ_F32 = 0, RSQ_F16 = 1, RSQ_BF16 = 2 };
/* rsq_state_alloc modes. */
enum { RSQ_INIT_ZERO = 0, RSQ_ATTACH = 1 };
/* Device status bits (rsq_get_status). */
enum {
  RSQ_F_NONFINITE = 1,       /* a non-finite value reached the state or the output */
  RSQ_F_SCALE_OVERFLOW = 2,  /* a step size overflowed binary16 */
  RSQ_F_CLIPPED = 4          /* a code was clamped to the code range */
};

/*
 * Configuration. All fields are read at rsq_state_alloc and copied.
 *
 *  abi_version     must be RSQ_ABI_VERSION
 *  model           RSQ_RETNET | RSQ_MAMBA2 | RSQ_GLA | RSQ_GDN
 *  batch, heads    tiles are (b, h) pairs, b-major; inputs are [batch][heads][.]
 *  d_k, d_v        per-head state is d_k x d_v (rows = key channels)
 *  group           scale group size along d_v: 8, 16, 32, 64 or 128, dividing d_v
 *  bits            4, 6, 8, or 32 (32 = unquantized fp32 state, the comparator
 *                  of "FP32 states"); ignored when head_bits != NULL
 *  head_bits       NULL, or host array [heads] of per-head widths in {4, 6, 8}
 *  scale_mode      RSQ_SCALE_DYNAMIC | RSQ_SCALE_PERSISTENT | RSQ_SCALE_YOKED
 *  scale_dtype     RSQ_F32 | RSQ_F16 (storage of the per-group step size)
 *  persist_trigger persistent step grows when absmax > trigger * qmax * s (> 0)
 *  bdr, bdr_eps    Bounded Directional Rounding on/off; a reversed element moves
 *                  one code toward its update when the new error stays within
 *                  (0.5 + bdr_eps) * s (bdr_eps >= 0.5 corrects every reversal
 *                  whose corrected code is inside the code range)
 *  lrb_k, lrb_m    Low-Rank Bypass: k residual columns kept by a merge, a merge
 *                  every m steps (capacity k + m fp16 column pairs); m = 0 = off.
 *                  Every update goes into the bypass as one column pair
 *                  (fp16(k), fp16(w)) and the codes only decay between merges.
 *                  With GDN the delta rule reads the stored state plus the
 *                  bypass: u = s_hat^T k + W (U^T k) ("Preserving Updates ...",
 *                  Table 6 GDN row, Tables 7 and 8)
 *  lrb_eps         merge threshold eps_L: |L_ij| > eps_L * s moves into the state
 *  gamma           RetNet only: host array [heads] of decays; NULL otherwise
 *  in_dtype        RSQ_F32 | RSQ_BF16: element type of q, k, v
 *  hadamard        0, or 1 for the INT4+Had baseline of "Preserving Updates",
 *                  Table 2: codes and steps describe each scale group of a
 *                  row rotated by the g x g Sylvester-Hadamard matrix H
 *                  (entries +-1): y = x H is what is quantized, and the state
 *                  reads back as (c s) H / g. Quantized widths with dynamic or
 *                  persistent scales only: no BDR, bypass or yoked scales
 *  pw_window       0, or W in [1, 16]: Gated DeltaNet pure-write window
 *                  ("Low-Bit GDN Recurrent-State Quantization: Global
 *                  Gradient-aware Allocation and Pure-Write Sliding Windows",
 *                  abstract). The state is the low-bit history H plus the last
 *                  W writes as FP8 (OCP E4M3, saturating) pairs (u, w) =
 *                  (k_t, beta_t v_t), slot (t - 1) mod W. Each step the pairs
 *                  that stay take the transition u <- alpha (u - beta k (k^T u)).
 *                  H takes it alone (the delta-rule step with v = 0); the pair
 *                  written W steps earlier takes it too, unrounded, and joins
 *                  H after it, x = H' + u' w^T, before requantization. Then
 *                  o_t = x^T q + sum_c w_c (u_c^T q). Quantized widths with
 *                  dynamic or persistent scales only
 *
 * Supported shapes (others return RSQ_E_UNSUPPORTED): d_v a multiple of
 * 8 * max(4, group / 8); d_k a multiple of 512 / max(4, group / 8) rows per
 * wavefront (128 for group <= 32, 64 for group 64, 32 for group 128) with
 * d_k * d_v <= 32768; GDN needs d_k to be a power of two; yoked scales run
 * without a bypass.
 */
typedef struct rsq_config {
  uint32_t abi_version;
  int32_t model, batch, heads, d_k, d_v;
  int32_t group;
  int32_t bits;
  const int32_t* head_bits;
  int32_t scale_mode, scale_dtype;
  float persist_trigger;
  int32_t bdr;
  float bdr_eps;
  int32_t lrb_k, lrb_m;
  float lrb_eps;
  const float* gamma;
  int32_t in_dtype;
  int32_t hadamard;
  int32_t pw_window;
} rsq_config;

typedef struct rsq_state rsq_state;  /* opaque host handle */

/*
 * Byte layout of a state buffer (all offsets from the buffer start; the
 * buffer must be 256-byte aligned).
 *
 *   [0, 256)            header: u32 magic 'RSQ1', u32 abi version, u64 config
 *                       hash, i64 step count t, i32 bypass fill n; the u32
 *                       device status word sits at byte 128
 *   head_table          heads x 32 bytes {i32 bits, f32 gamma, u64 tile offset
 *                       inside a batch row, u32 scales, bypass_u, bypass_w and
 *                       ref section offsets inside the tile (codes at 0)}
 *   tile (b, h)         at tiles + b * batch_stride + head_offset[h]; inside a
 *                       tile, sections at the offsets below (each 256-aligned):
 *     codes   d_k*d_v*bits/8 bytes in 8x8 chunks. Chunk (rb, cb) (row block
 *             rb = i/8, column block cb = j/8) starts at
 *             (cb * d_k/8 + rb) * 8 * bits bytes. Inside a chunk, row r:
 *               bits 4: u32 word r; byte c (c < 4) holds column c in bits 0-3
 *                       and column c+4 in bits 4-7
 *               bits 8: bytes 8r .. 8r+7 hold columns 0..7
 *               bits 6: code = 4*hi + lo, hi a signed nibble stored like
 *                       bits 4 in the first 32 bytes, lo in [0,3] in the last
 *                       16 bytes: u32 word p holds rows 2p and 2p+1, byte c
 *                       = lo(2p,c) | lo(2p,c+4)<<2 | lo(2p+1,c)<<4 | lo(2p+1,c+4)<<6
 *               bits 32: floats 8r .. 8r+7 hold columns 0..7
 *             4/6/8-bit codes are two's complement, in [-2^(b-1), 2^(b-1)-1].
 *     scales  [d_v/group][d_k] step sizes (scale_dtype); value = code * step
 *     bypass_u [k+m][d_k] fp16 (column c contiguous), bypass_w [k+m][d_v] fp16;
 *             with a pure-write window the same sections hold u [W][d_k] and
 *             w [W][d_v] as E4M3 bytes
 *     ref     yoked reference state, fp32, chunk layout as bits 32
 */
typedef struct rsq_layout {
  size_t header;        /* 0 */
  size_t status;        /* byte offset of the u32 status word */
  size_t head_table;
  size_t tiles;         /* start of tile (0, 0) */
  size_t batch_stride;  /* bytes between tiles (b, h) and (b+1, h) */
  size_t tile_codes;    /* section offsets inside a tile of head h are given by */
  size_t tile_scales;   /*   rsq_tile_sections(); these fields hold head 0's */
  size_t tile_bypass_u;
  size_t tile_bypass_w;
  size_t tile_ref;
  size_t total;         /* == rsq_state_bytes */
} rsq_layout;

/* Bytes the caller must allocate for cfg. */
rsq_status rsq_state_bytes(const rsq_config* cfg, size_t* bytes);

/*
 * Bind a caller-owned device buffer (>= rsq_state_bytes, 256-byte aligned) to
 * a new handle. RSQ_INIT_ZERO clears the buffer (codes 0, steps 0, empty
 * bypass, zero reference: the initial state) and writes the header, stream-
 * ordered. RSQ_ATTACH keeps the contents (a saved state) after checking the
 * header's magic, version and config hash, and restores t and n from it; it
 * synchronizes `stream`. The buffer must stay alive until rsq_state_free.
 */
rsq_status rsq_state_alloc(const rsq_config* cfg, void* dev_buf, size_t buf_bytes,
                           int32_t init, void* stream, rsq_state** out);

/* Free the host handle (not the device buffer). NULL is accepted. */
rsq_status rsq_state_free(rsq_state* st);

/* Layout of the bound buffer (host struct, filled by the call). */
rsq_status rsq_state_layout(const rsq_state* st, rsq_layout* out);

/* Section offsets of a tile of head h, relative to the tile start, and the
 * tile's offset inside a batch row. Any pointer may be NULL. */
rsq_status rsq_tile_sections(const rsq_state* st, int32_t head, size_t* head_offset,
                             size_t* codes, size_t* scales, size_t* bypass_u,
                             size_t* bypass_w, size_t* ref, int32_t* bits);

/* Host-side step count t and bypass fill n of the handle. */
rsq_status rsq_state_counters(const rsq_state* st, int64_t* t, int32_t* n);

/*
 * One decode step of every tile, in place.
 *   q, k  device [batch][heads][d_k] of in_dtype;  v device [batch][heads][d_v]
 *   alpha device fp32: NULL for RetNet; [batch][heads] for Mamba2 and GDN;
 *         [batch][heads][d_k] for GLA (per key channel)
 *   beta  device fp32 [batch][heads], GDN only (NULL otherwise)
 *   o     device fp32 [batch][heads][d_v], written: o_t = S_t^T q_t from the
 *         updated state before requantization (plus W (U^T q) with a bypass)
 * Inputs must be contiguous and 16-byte aligned. With a bypass, returns
 * RSQ_E_BYPASS_FULL once k+m columns are in use (call rsq_merge_bypass).
 * Steps of states without a bypass or window can be captured in a HIP graph
 * and replayed; with a bypass or a pure-write window the step's column or
 * slot comes from the host handle, so such a step (and rsq_merge_bypass)
 * returns RSQ_E_UNSUPPORTED while `stream` is capturing.
 */
rsq_status rsq_decode_step(rsq_state* st, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, float* o, void* stream);

/*
 * rsq_decode_step for profiling: the step's decode kernel records
 * start_event (a hipEvent_t, may be NULL) when it begins and stop_event when
 * it ends. The timestamps come from the kernel's own dispatch, so no extra
 * command enters the stream and back-to-back steps stay back to back. The
 * events belong to the caller and must exist on the stream's device.
 */
rsq_status rsq_decode_step_timed(rsq_state* st, const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta, float* o, void* stream,
                                 void* start_event, void* stop_event);

/*
 * rsq_decode_step with error accounting ("Preserving Updates ...", Fig. 1:
 * per-step rounding errors R and their decayed sum E_T; Fig. 2: the coherent
 * gain g_T and its parts on lost and moved updates; Fig. 4: lost, moved and
 * reversed updates; Table 5: |b| / step and the lost fraction). The state
 * advances exactly as rsq_decode_step would (same codes, steps and o). Per
 * element of each tile, with b = fl(k_i w_j) the element's update B_t,
 * s' the step after the scale rule, x the value before rounding, r the
 * no-update value fl(c fl(a s)) and c the stored code:
 *   R = fl(c s' - x); lost: b != 0 and c equals the code r rounds to on the
 *   same grid; moved: b != 0 and not lost; reversed: b != 0 and c s' lies
 *   strictly on the other side of r from b.
 *   acc    device fp32 [tiles][6][d_k*d_v], each plane in the bits-32 chunk
 *          layout of the codes (tiles b-major): E, D, E_lost, D_lost, E_moved,
 *          D_moved, updated in place with a = the row decay of Table 1:
 *          E <- fl(fl(a E) + R_m), D <- fl(fl(fl(a a) D) + fl(R_m R_m)),
 *          R_m = R on the plane's mask (all, lost, moved), 0 elsewhere.
 *          Zero it to start a window; g_T = sum E^2 / sum D.
 *   ratio  device fp32 [tiles][d_k*d_v] (chunk layout) or NULL: this step's
 *          fl(|b| RN(1/s')) for updated elements with a finite s' > 0, else -1
 *   counts device u32 [tiles][4]: updated, lost, moved, reversed, added to
 * Buffers are 16-byte aligned and owned by the caller. Returns
 * RSQ_E_UNSUPPORTED for fp32 states, a bypass or yoked scales.
 */
rsq_status rsq_decode_step_diag(rsq_state* st, const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, float* o, float* acc,
                                float* ratio, uint32_t* counts, void* stream);

/*
 * Low-Rank Bypass merge: L = U W^T; elements with |L_ij| > eps_L * s move
 * into the quantized state, which is requantized (with BDR when enabled,
 * toward sign(L_ij)); the rest is replaced by a rank-k approximation kept as
 * k fp16 column pairs. Sets n = k. RSQ_E_NO_BYPASS without a bypass.
 */
rsq_status rsq_merge_bypass(rsq_state* st, void* stream);

/* rsq_merge_bypass for profiling: the merge kernel's dispatch records
 * start_event / stop_event (hipEvent_t, either may be NULL), as in
 * rsq_decode_step_timed. */
rsq_status rsq_merge_bypass_timed(rsq_state* st, void* stream, void* start_event, void* stop_event);

/* o = deq(S)^T q (+ W (U^T q)); reads the state only. q as in decode_step. */
rsq_status rsq_readout(const rsq_state* st, const void* q, float* o, void* stream);

/* Synchronize `stream`, then return and clear the device status bits. */
rsq_status rsq_get_status(rsq_state* st, uint32_t* flags, void* stream);

/*
 * Decay-aware per-head widths (host only; "Low-Bit Recurrent States in Hybrid
 * Language Models", abstract: Gramian distortion weights and normalised state
 * ranges). Head h at width b costs w_h / (2^(b-1) - 1)^2 with
 * w_h = range[h]^2 / (1 - decay_sq[h]): 1 / (1 - E[a^2]) is how much of an
 * injected error a state decaying by a_t keeps over the future steps. The
 * widths {4, 6, 8} written to bits_out (host array [heads]) minimise the total
 * cost with sum(bits) <= floor(mean_bits * heads); ties go to the lower head
 * index, and a head gains width only where that lowers the cost.
 *   decay_sq  host [heads]: E[a_t^2] of the head's decay, in [0, 1)
 *             (GLA: the mean over key channels of E[a_t,i^2])
 *   range     host [heads]: the head's typical group absmax (>= 0, finite)
 *   mean_bits in [4, 8]
 * Returns RSQ_E_INVALID on a bad argument (bits_out is then unspecified).
 * The result can be passed as rsq_config.head_bits.
 */
rsq_status rsq_allocate_head_bits(const float* decay_sq, const float* range, int32_t heads,
                                  float mean_bits, int32_t* bits_out);

/* Thread-local description of the last error (never NULL). */
const char* rsq_last_error(void);

int32_t rsq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RSQ_H */
