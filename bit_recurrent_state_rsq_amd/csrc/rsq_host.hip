// Host side of the C ABI declared in include/rsq.h: validation, state layout,
// the handle (step count t, bypass fill n), kernel selection and launch on the
// caller's stream, status word and error strings.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <map>
#include <tuple>
#include <string>
#include <utility>
#include <vector>

#include "rsq.h"
#include "rsq_kernels.hpp"

using rsq::HeadEntry;
using rsq::StepArgs;

namespace {

thread_local std::string g_err = "no error";

rsq_status fail(rsq_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

rsq_status hip_fail(hipError_t e, const char* what) {
  return fail(RSQ_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr uint32_t kMagicHdr = 0x31515352u;  // 'RSQ1'
constexpr size_t kAlign = 256;
constexpr size_t kHeaderBytes = 256;
constexpr size_t kStatusOff = 128;
constexpr size_t kHdrT = 16, kHdrN = 24;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Geometry {
  int cl, wr, wc, wrw, wcw, threads;
  size_t lds;         // decode / readout
  size_t lds_merge;   // bypass merge (0 without a bypass)
  int merge_chunk;    // basis columns per merge product pass
};

constexpr size_t kLdsBytes = 160 * 1024;   // LDS of one gfx950 compute unit

uint64_t fnv1a(uint64_t h, const void* p, size_t n) {
  const uint8_t* b = static_cast<const uint8_t*>(p);
  for (size_t i = 0; i < n; ++i) {
    h ^= b[i];
    h *= 1099511628211ull;
  }
  return h;
}

}  // namespace

struct rsq_state {
  rsq_config cfg;
  std::vector<int32_t> head_bits;
  std::vector<float> gamma;
  uint8_t* buf = nullptr;
  size_t bytes = 0;
  rsq_layout layout{};
  std::vector<HeadEntry> heads;
  HeadEntry* dev_heads = nullptr;
  int64_t t = 0;
  int32_t n = 0;
  int32_t cap = 0;
  int32_t pw = 0;       // pure-write window size W (0 = none)
  bool uniform = false; // every head's table entry alike up to its offset
  bool bypass = false;
  bool all32 = false;
  int max_bits = 0;     // widest head: a decode wavefront stages 512 bytes per code bit in LDS
  uint64_t hash = 0;
  Geometry geo{};
};

namespace {

// Full description of a configuration: validation, per-head bits, layout.
struct Plan {
  std::vector<int32_t> bits;
  std::vector<float> gamma;
  std::vector<HeadEntry> heads;
  rsq_layout layout{};
  Geometry geo{};
  int cap = 0;
  int pw = 0;
  bool bypass = false, all32 = false;
  uint64_t hash = 0;
};

rsq_status make_plan(const rsq_config* c, Plan& p) {
  if (!c) return fail(RSQ_E_INVALID, "cfg is NULL");
  if (c->abi_version != RSQ_ABI_VERSION)
    return fail(RSQ_E_INVALID, "abi_version %u, library is %d", c->abi_version, RSQ_ABI_VERSION);
  if (c->model < RSQ_RETNET || c->model > RSQ_GDN) return fail(RSQ_E_INVALID, "model %d", c->model);
  if (c->batch < 1 || c->heads < 1) return fail(RSQ_E_INVALID, "batch %d heads %d", c->batch, c->heads);
  if (c->d_k < 8 || c->d_v < 8 || c->d_k % 8 || c->d_v % 8)
    return fail(RSQ_E_INVALID, "d_k %d d_v %d must be positive multiples of 8", c->d_k, c->d_v);
  const int g = c->group;
  if (g != 8 && g != 16 && g != 32 && g != 64 && g != 128)
    return fail(RSQ_E_INVALID, "group %d not in {8,16,32,64,128}", g);
  if (c->d_v % g) return fail(RSQ_E_INVALID, "group %d does not divide d_v %d", g, c->d_v);
  if (c->scale_mode < RSQ_SCALE_DYNAMIC || c->scale_mode > RSQ_SCALE_YOKED)
    return fail(RSQ_E_INVALID, "scale_mode %d", c->scale_mode);
  if (c->scale_dtype != RSQ_F32 && c->scale_dtype != RSQ_F16)
    return fail(RSQ_E_INVALID, "scale_dtype %d", c->scale_dtype);
  if (c->in_dtype != RSQ_F32 && c->in_dtype != RSQ_BF16) return fail(RSQ_E_INVALID, "in_dtype %d", c->in_dtype);
  if (c->scale_mode == RSQ_SCALE_PERSISTENT && !(c->persist_trigger > 0.f && std::isfinite(c->persist_trigger)))
    return fail(RSQ_E_INVALID, "persist_trigger must be finite and > 0");
  if (c->bdr && !(c->bdr_eps >= 0.f && std::isfinite(c->bdr_eps)))
    return fail(RSQ_E_INVALID, "bdr_eps must be finite and >= 0");
  if (c->lrb_k < 0 || c->lrb_m < 0) return fail(RSQ_E_INVALID, "lrb_k %d lrb_m %d", c->lrb_k, c->lrb_m);
  if (c->lrb_m == 0 && c->lrb_k != 0) return fail(RSQ_E_INVALID, "lrb_k > 0 needs lrb_m > 0");
  if (c->lrb_m > 0 && !(c->lrb_eps >= 0.f)) return fail(RSQ_E_INVALID, "lrb_eps must be >= 0");
  if ((c->model == RSQ_RETNET) != (c->gamma != nullptr))
    return fail(RSQ_E_INVALID, "gamma must be given for RetNet and only for RetNet");

  p.bits.resize(c->heads);
  for (int h = 0; h < c->heads; ++h) {
    const int b = c->head_bits ? c->head_bits[h] : c->bits;
    if (c->head_bits ? (b != 4 && b != 6 && b != 8) : (b != 4 && b != 6 && b != 8 && b != 32))
      return fail(RSQ_E_INVALID, "bits %d for head %d", b, h);
    p.bits[h] = b;
  }
  p.all32 = !c->head_bits && c->bits == 32;
  p.bypass = c->lrb_m > 0;
  p.cap = p.bypass ? c->lrb_k + c->lrb_m : 0;
  const bool yoked = c->scale_mode == RSQ_SCALE_YOKED && !p.all32;
  if (p.all32 && (p.bypass || c->bdr))
    return fail(RSQ_E_INVALID, "bits 32 (fp32 state) takes no bypass and no BDR");
  if (p.bypass && yoked) return fail(RSQ_E_UNSUPPORTED, "yoked scales with a bypass are not implemented");
  if (p.cap > rsq::kMaxCap) return fail(RSQ_E_UNSUPPORTED, "bypass capacity %d > %d", p.cap, rsq::kMaxCap);
  if (c->hadamard != 0 && c->hadamard != 1) return fail(RSQ_E_INVALID, "hadamard %d", c->hadamard);
  if (c->pw_window < 0 || c->pw_window > 16) return fail(RSQ_E_INVALID, "pw_window %d not in [0, 16]", c->pw_window);
  if (c->pw_window) {
    if (c->model != RSQ_GDN) return fail(RSQ_E_UNSUPPORTED, "the pure-write window is a Gated DeltaNet option");
    if (p.all32 || p.bypass || c->bdr || c->hadamard || c->scale_mode == RSQ_SCALE_YOKED)
      return fail(RSQ_E_UNSUPPORTED,
                  "the pure-write window runs on quantized states without BDR, bypass, rotation or yoked scales");
    if (c->d_k > 1024) return fail(RSQ_E_UNSUPPORTED, "the pure-write window needs d_k <= 1024");
    p.pw = c->pw_window;
    p.cap = p.pw;
  }
  if (c->hadamard && (p.all32 || p.bypass || c->bdr || c->scale_mode == RSQ_SCALE_YOKED))
    return fail(RSQ_E_UNSUPPORTED, "the Hadamard rotation runs on quantized states without BDR, bypass or yoked scales");

  // work decomposition
  Geometry& G = p.geo;
  G.cl = std::max(4, g / 8);
  G.wr = 512 / G.cl;
  G.wc = 8 * G.cl;
  if (c->d_v % G.wc) return fail(RSQ_E_UNSUPPORTED, "d_v %d must be a multiple of %d for group %d", c->d_v, G.wc, g);
  if (c->d_k % G.wr) return fail(RSQ_E_UNSUPPORTED, "d_k %d must be a multiple of %d for group %d", c->d_k, G.wr, g);
  G.wrw = c->d_k / G.wr;
  G.wcw = c->d_v / G.wc;
  G.threads = 64 * G.wrw * G.wcw;
  if (G.threads > 512) return fail(RSQ_E_UNSUPPORTED, "d_k*d_v = %d exceeds 32768", c->d_k * c->d_v);
  if (c->model == RSQ_GDN && (c->d_k & (c->d_k - 1)))
    return fail(RSQ_E_UNSUPPORTED, "the delta rule needs a power-of-two d_k, got %d", c->d_k);
  // per-wave w broadcast, 2 x retrieval partials, readout partials, bypass
  // projections; with a bypass also the delta rule's U^T k and W (U^T k)
  G.lds = (size_t)((G.threads / 64) * G.wc + 3 * G.wrw * c->d_v + rsq::kMaxCap * (1 + G.threads / 64) +
                   (p.bypass ? rsq::kMaxCap + c->d_v : 0)) *
              sizeof(float) +
          (p.bypass && c->model == RSQ_GDN ? (size_t)(rsq::gdn_wstage_bytes(c->d_v) + rsq::gdn_ustage_bytes(c->d_k)) : 0);
  // the merge's closing products with R take 8 columns per pass (at most 8
  // columns are kept in the common case), which keeps its LDS small enough
  // for two tiles per compute unit on 128 x 128 heads
  G.merge_chunk = 8;
  G.lds_merge = p.bypass ? rsq::merge_lds_floats(c->d_k, c->d_v, G.wrw, G.wcw, p.cap, c->lrb_k, 8) * sizeof(float) : 0;
  if (G.lds_merge > kLdsBytes)
    return fail(RSQ_E_UNSUPPORTED, "the bypass merge of a %d x %d tile with %d columns needs %zu bytes of LDS",
                c->d_k, c->d_v, p.cap, G.lds_merge);

  // layout
  if (c->gamma) {
    p.gamma.assign(c->gamma, c->gamma + c->heads);
    for (float v : p.gamma)
      if (!std::isfinite(v)) return fail(RSQ_E_INVALID, "gamma must be finite");
  }
  rsq_layout& L = p.layout;
  L.header = 0;
  L.status = kStatusOff;
  L.head_table = kHeaderBytes;
  L.tiles = align_up(kHeaderBytes + sizeof(HeadEntry) * (size_t)c->heads);
  p.heads.resize(c->heads);
  size_t off = 0;
  const size_t sbytes = c->scale_dtype == RSQ_F16 ? 2 : 4;
  for (int h = 0; h < c->heads; ++h) {
    HeadEntry& e = p.heads[h];
    e.bits = p.bits[h];
    e.gamma = c->gamma ? c->gamma[h] : 0.f;
    e.head_offset = off;
    const size_t codes = (size_t)c->d_k * c->d_v * e.bits / 8;
    const size_t scales = e.bits == 32 ? 0 : (size_t)(c->d_v / g) * c->d_k * sbytes;
    const size_t pair_bytes = p.pw ? 1 : 2;   // E4M3 window pairs, fp16 bypass columns
    const size_t bu = (size_t)p.cap * c->d_k * pair_bytes, bw = (size_t)p.cap * c->d_v * pair_bytes;
    const size_t ref = yoked ? (size_t)c->d_k * c->d_v * 4 : 0;
    size_t o = align_up(codes);
    e.scales = (uint32_t)o;
    o += align_up(scales);
    e.bypass_u = (uint32_t)o;
    o += align_up(bu);
    e.bypass_w = (uint32_t)o;
    o += align_up(bw);
    e.ref = (uint32_t)o;
    o += align_up(ref);
    off += o;
  }
  L.batch_stride = off;
  L.tile_codes = 0;
  L.tile_scales = p.heads[0].scales;
  L.tile_bypass_u = p.heads[0].bypass_u;
  L.tile_bypass_w = p.heads[0].bypass_w;
  L.tile_ref = p.heads[0].ref;
  L.total = L.tiles + (size_t)c->batch * L.batch_stride;

  // identity of the configuration (for RSQ_ATTACH)
  uint64_t hsh = 1469598103934665603ull;
  const int32_t ints[] = {c->model, c->batch, c->heads, c->d_k, c->d_v, g, c->scale_mode, c->scale_dtype,
                          c->bdr, c->lrb_k, c->lrb_m, c->in_dtype};
  hsh = fnv1a(hsh, ints, sizeof ints);
  hsh = fnv1a(hsh, p.bits.data(), p.bits.size() * 4);
  const float fl[] = {c->scale_mode == RSQ_SCALE_PERSISTENT ? c->persist_trigger : 0.f,
                      c->bdr ? c->bdr_eps : 0.f, p.bypass ? c->lrb_eps : 0.f};
  hsh = fnv1a(hsh, fl, sizeof fl);
  if (!p.gamma.empty()) hsh = fnv1a(hsh, p.gamma.data(), p.gamma.size() * 4);
  if (c->hadamard) hsh = fnv1a(hsh, "hadamard", 8);
  if (p.pw) hsh = fnv1a(hsh, &p.pw, sizeof p.pw);
  p.hash = hsh;
  return RSQ_OK;
}

__global__ void fill_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

__global__ void clear_word_kernel(uint32_t* p) { *p = 0u; }

StepArgs base_args(rsq_state* st) {
  StepArgs a{};
  a.tiles = st->buf + st->layout.tiles;
  a.heads = reinterpret_cast<const HeadEntry*>(st->buf + st->layout.head_table);
  a.status = reinterpret_cast<uint32_t*>(st->buf + st->layout.status);
  a.hdr_t = reinterpret_cast<int64_t*>(st->buf + kHdrT);
  a.hdr_n = reinterpret_cast<int32_t*>(st->buf + kHdrN);
  a.batch_stride = st->layout.batch_stride;
  a.H = st->cfg.heads;
  a.dk = st->cfg.d_k;
  a.dv = st->cfg.d_v;
  a.group = st->cfg.group;
  a.smode = st->all32 ? rsq::kScaleDynamic : st->cfg.scale_mode;
  a.trigger = st->cfg.persist_trigger;
  a.bdr = st->cfg.bdr;
  a.bdr_eps = st->cfg.bdr_eps;
  a.bypass = st->bypass ? 1 : 0;
  a.n = st->n;
  a.cap = st->cap;
  a.lrb_k = st->cfg.lrb_k;
  a.lrb_eps = st->cfg.lrb_eps;
  a.in_bf16 = st->cfg.in_dtype == RSQ_BF16;
  a.scale_f16 = st->cfg.scale_dtype == RSQ_F16;
  a.hadamard = st->cfg.hadamard;
  a.pw = st->pw;
  a.merge_chunk = st->geo.merge_chunk;
  a.uniform = st->uniform ? 1 : 0;
  if (st->uniform) {
    a.uni = st->heads[0];
    a.uni_stride = st->heads.size() > 1 ? st->heads[1].head_offset : 0;
  }
  return a;
}

// Whether all `blocks` workgroups of fn are resident on the current device at
// once (occupancy per CU times the CU count), cached per device, kernel, block
// size and LDS size. A failed query answers no.
bool one_round(rsq::DecodeFn fn, unsigned blocks, unsigned threads, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, unsigned, size_t>, long> resident;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const auto key = std::make_tuple(dev, reinterpret_cast<const void*>(fn), threads, lds);
  std::lock_guard<std::mutex> lock(mu);
  auto it = resident.find(key);
  if (it == resident.end()) {
    int per_cu = 0, cus = 0;
    long n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), (int)threads, lds) ==
            hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      n = (long)per_cu * cus;
    (void)hipGetLastError();   // a failed query leaves no error for the launch to report
    it = resident.emplace(key, n).first;
  }
  return (long)blocks <= it->second;
}

// The step count t and the bypass fill n (or the window's pair count) live in
// the host handle and reach the kernels as launch arguments, so a graph
// captured from such a step would replay the same column and slot every
// time. Steps that read them are refused while the stream is capturing.
rsq_status refuse_capture(void* stream, const char* what) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing((hipStream_t)stream, &cap);
  if (e != hipSuccess) return hip_fail(e, "stream capture query");
  if (cap != hipStreamCaptureStatusNone)
    return fail(RSQ_E_UNSUPPORTED, "%s cannot be captured in a graph: its launch arguments change every call", what);
  return RSQ_OK;
}

rsq_status launch(rsq::DecodeFn fn, const rsq_state* st, const StepArgs& a, void* stream,
                  void* ev_start = nullptr, void* ev_stop = nullptr, size_t lds = 0) {
  const dim3 grid(st->cfg.batch * st->cfg.heads), block(st->geo.threads);
  if (lds == 0) lds = st->geo.lds;
  // a grid resident at once runs the raised-priority twin, where there is one
  if (rsq::DecodeFn twin = rsq::decode_boost_twin(fn))
    if (one_round(fn, grid.x, block.x, lds)) fn = twin;
  if (lds > 64 * 1024) {
    // raised once per kernel and device, to the largest size a launch has
    // asked for (the attribute call is host work that need not repeat every step)
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, size_t> raised;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "current device");
    const auto key = std::make_pair(dev, reinterpret_cast<const void*>(fn));
    std::lock_guard<std::mutex> lock(mu);
    auto it = raised.find(key);
    if (it == raised.end() || it->second < lds) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return hip_fail(e, "raising the kernel's LDS limit");
      raised[key] = lds;
    }
  }
  if (ev_start || ev_stop) {
    // the events ride on the dispatch packet itself: no marker enters the stream
    hipExtLaunchKernelGGL(fn, grid, block, (uint32_t)lds, (hipStream_t)stream, (hipEvent_t)ev_start,
                          (hipEvent_t)ev_stop, 0u, a);
  } else {
    hipLaunchKernelGGL(fn, grid, block, lds, (hipStream_t)stream, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return RSQ_OK;
}

}  // namespace

extern "C" {

int32_t rsq_abi_version(void) { return RSQ_ABI_VERSION; }

const char* rsq_last_error(void) { return g_err.c_str(); }

rsq_status rsq_state_bytes(const rsq_config* cfg, size_t* bytes) {
  if (!bytes) return fail(RSQ_E_INVALID, "bytes is NULL");
  Plan p;
  const rsq_status s = make_plan(cfg, p);
  if (s != RSQ_OK) return s;
  *bytes = p.layout.total;
  return RSQ_OK;
}

rsq_status rsq_state_alloc(const rsq_config* cfg, void* dev_buf, size_t buf_bytes, int32_t init, void* stream,
                           rsq_state** out) {
  if (!out) return fail(RSQ_E_INVALID, "out is NULL");
  *out = nullptr;
  Plan p;
  rsq_status s = make_plan(cfg, p);
  if (s != RSQ_OK) return s;
  if (!dev_buf) return fail(RSQ_E_INVALID, "dev_buf is NULL");
  if (reinterpret_cast<uintptr_t>(dev_buf) % kAlign) return fail(RSQ_E_INVALID, "dev_buf is not 256-byte aligned");
  if (buf_bytes < p.layout.total)
    return fail(RSQ_E_BUFFER, "buffer has %zu bytes, state needs %zu", buf_bytes, p.layout.total);
  if (init != RSQ_INIT_ZERO && init != RSQ_ATTACH) return fail(RSQ_E_INVALID, "init %d", init);

  rsq_state* st = new rsq_state();
  st->cfg = *cfg;
  st->head_bits = p.bits;
  st->gamma = p.gamma;
  st->cfg.head_bits = nullptr;   // copies live in the handle
  st->cfg.gamma = st->gamma.empty() ? nullptr : st->gamma.data();
  st->buf = static_cast<uint8_t*>(dev_buf);
  st->bytes = buf_bytes;
  st->layout = p.layout;
  st->heads = p.heads;
  st->cap = p.cap;
  st->pw = p.pw;
  st->bypass = p.bypass;
  st->uniform = true;
  for (size_t h = 1; h < p.heads.size(); ++h) {
    const HeadEntry& e0 = p.heads[0];
    const HeadEntry& e = p.heads[h];
    st->uniform = st->uniform && e.bits == e0.bits && e.gamma == e0.gamma && e.scales == e0.scales &&
                  e.bypass_u == e0.bypass_u && e.bypass_w == e0.bypass_w && e.ref == e0.ref &&
                  e.head_offset == (uint64_t)h * p.heads[1].head_offset;
  }
  st->all32 = p.all32;
  st->max_bits = 0;
  for (const HeadEntry& e : p.heads) st->max_bits = std::max(st->max_bits, (int)e.bits);
  st->hash = p.hash;
  st->geo = p.geo;
  hipStream_t hs = (hipStream_t)stream;

  std::vector<uint8_t> hdr(p.layout.tiles, 0);
  uint32_t magic = kMagicHdr, ver = RSQ_ABI_VERSION;
  std::memcpy(&hdr[0], &magic, 4);
  std::memcpy(&hdr[4], &ver, 4);
  std::memcpy(&hdr[8], &st->hash, 8);
  std::memcpy(&hdr[kHeaderBytes], p.heads.data(), p.heads.size() * sizeof(HeadEntry));

  hipError_t e;
  if (init == RSQ_INIT_ZERO) {
    const size_t n16 = p.layout.total / 16;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, hs, reinterpret_cast<uint4*>(dev_buf), n16);
    if ((e = hipGetLastError()) != hipSuccess) { delete st; return hip_fail(e, "zero fill"); }
    if ((e = hipMemcpyAsync(dev_buf, hdr.data(), hdr.size(), hipMemcpyHostToDevice, hs)) != hipSuccess) {
      delete st;
      return hip_fail(e, "header upload");
    }
    if ((e = hipStreamSynchronize(hs)) != hipSuccess) { delete st; return hip_fail(e, "stream sync"); }
  } else {
    std::vector<uint8_t> got(p.layout.tiles);
    if ((e = hipMemcpyAsync(got.data(), dev_buf, got.size(), hipMemcpyDeviceToHost, hs)) != hipSuccess ||
        (e = hipStreamSynchronize(hs)) != hipSuccess) {
      delete st;
      return hip_fail(e, "header download");
    }
    uint32_t gm, gv;
    uint64_t gh;
    std::memcpy(&gm, &got[0], 4);
    std::memcpy(&gv, &got[4], 4);
    std::memcpy(&gh, &got[8], 8);
    if (gm != kMagicHdr || gv != RSQ_ABI_VERSION || gh != st->hash ||
        std::memcmp(&got[kHeaderBytes], &hdr[kHeaderBytes], p.heads.size() * sizeof(HeadEntry)) != 0) {
      delete st;
      return fail(RSQ_E_ATTACH, "buffer header does not match this configuration");
    }
    std::memcpy(&st->t, &got[kHdrT], 8);
    std::memcpy(&st->n, &got[kHdrN], 4);
    if (st->n < 0 || st->n > st->cap) {
      delete st;
      return fail(RSQ_E_ATTACH, "bypass fill %d out of range", st->n);
    }
  }
  *out = st;
  return RSQ_OK;
}

rsq_status rsq_state_free(rsq_state* st) {
  delete st;
  return RSQ_OK;
}

rsq_status rsq_state_layout(const rsq_state* st, rsq_layout* out) {
  if (!st || !out) return fail(RSQ_E_INVALID, "NULL argument");
  *out = st->layout;
  return RSQ_OK;
}

rsq_status rsq_tile_sections(const rsq_state* st, int32_t head, size_t* head_offset, size_t* codes,
                             size_t* scales, size_t* bypass_u, size_t* bypass_w, size_t* ref, int32_t* bits) {
  if (!st) return fail(RSQ_E_INVALID, "state is NULL");
  if (head < 0 || head >= st->cfg.heads) return fail(RSQ_E_INVALID, "head %d out of range", head);
  const HeadEntry& e = st->heads[head];
  if (head_offset) *head_offset = e.head_offset;
  if (codes) *codes = 0;
  if (scales) *scales = e.scales;
  if (bypass_u) *bypass_u = e.bypass_u;
  if (bypass_w) *bypass_w = e.bypass_w;
  if (ref) *ref = e.ref;
  if (bits) *bits = e.bits;
  return RSQ_OK;
}

rsq_status rsq_state_counters(const rsq_state* st, int64_t* t, int32_t* n) {
  if (!st) return fail(RSQ_E_INVALID, "state is NULL");
  if (t) *t = st->t;
  if (n) *n = st->n;
  return RSQ_OK;
}

rsq_status rsq_decode_step(rsq_state* st, const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, float* o, void* stream) {
  return rsq_decode_step_timed(st, q, k, v, alpha, beta, o, stream, nullptr, nullptr);
}

}  // extern "C"

namespace {

struct DiagBuffers {
  float* acc;
  float* ratio;
  uint32_t* counts;
};

rsq_status decode_step(rsq_state* st, const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, float* o, void* stream, void* start_event, void* stop_event,
                       const DiagBuffers* dg) {
  if (!st) return fail(RSQ_E_INVALID, "state is NULL");
  if (!q || !k || !v || !o) return fail(RSQ_E_INVALID, "q, k, v and o must be non-NULL");
  const int model = st->cfg.model;
  if (model == RSQ_RETNET && alpha) return fail(RSQ_E_INVALID, "RetNet takes no alpha");
  if (model != RSQ_RETNET && !alpha) return fail(RSQ_E_INVALID, "alpha is required for this model");
  if ((model == RSQ_GDN) != (beta != nullptr)) return fail(RSQ_E_INVALID, "beta is required for GDN only");
  const void* ptrs[] = {q, k, v, alpha, beta, o};
  for (const void* ptr : ptrs)
    if (ptr && reinterpret_cast<uintptr_t>(ptr) % 16) return fail(RSQ_E_INVALID, "inputs must be 16-byte aligned");
  if (st->bypass && st->n >= st->cap)
    return fail(RSQ_E_BYPASS_FULL, "bypass holds %d of %d columns: call rsq_merge_bypass", st->n, st->cap);
  if (st->bypass || st->pw) {
    const rsq_status cs = refuse_capture(stream, "a decode step of a state with a bypass or a pure-write window");
    if (cs != RSQ_OK) return cs;
  }
  StepArgs a = base_args(st);
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.o = o;
  a.t_next = st->t + 1;
  int feat = rsq::kFeatPlain;
  if (st->all32) feat = rsq::kFeatF32;
  else if (st->bypass) feat = rsq::kFeatBypass;
  else if (st->cfg.scale_mode == RSQ_SCALE_YOKED) feat = rsq::kFeatYoked;
  else if (st->cfg.bdr) feat = rsq::kFeatBdr;
  else if (st->cfg.hadamard) feat = rsq::kFeatHad;
  else if (st->pw) feat = rsq::kFeatPW;
  if (dg) {
    if (feat != rsq::kFeatPlain && feat != rsq::kFeatBdr)
      return fail(RSQ_E_UNSUPPORTED,
                  "error accounting runs on quantized states without a bypass, yoked scales or a rotation");
    if (!dg->acc || !dg->counts) return fail(RSQ_E_INVALID, "acc and counts must be non-NULL");
    if (reinterpret_cast<uintptr_t>(dg->acc) % 16 || reinterpret_cast<uintptr_t>(dg->ratio) % 16 ||
        reinterpret_cast<uintptr_t>(dg->counts) % 16)
      return fail(RSQ_E_INVALID, "accounting buffers must be 16-byte aligned");
    feat = rsq::kFeatDiag;
    a.dg_acc = dg->acc;
    a.dg_ratio = dg->ratio;
    a.dg_counts = dg->counts;
  }
  // compile-time specialisations of (scale mode, step dtype, input dtype)
  const bool sf16 = st->cfg.scale_dtype == RSQ_F16, bf16 = st->cfg.in_dtype == RSQ_BF16;
  const int sm = st->cfg.scale_mode;
  const int g = st->cfg.group;
  int spec = 0;
  if (sm == RSQ_SCALE_PERSISTENT && sf16 && bf16 && g == 32) spec = 1;
  else if (sm == RSQ_SCALE_DYNAMIC && !sf16 && bf16 && g == 64) spec = 2;
  else if (sm == RSQ_SCALE_DYNAMIC && sf16 && bf16 && g == 32) spec = 3;
  else if (sm == RSQ_SCALE_DYNAMIC && !sf16 && !bf16 && g == 64) spec = 4;
  rsq::DecodeFn fn = rsq::decode_kernel_for(model, st->geo.cl, feat, spec);
  // quantized states without a bypass: every wavefront stages its code
  // chunks in LDS (512 bytes per code bit), after the step's own areas
  size_t lds = 0;
  if (!st->all32 && !st->bypass) {
    const size_t stage = (st->geo.lds + 15) & ~(size_t)15;
    a.lds_stage = (int32_t)stage;
    lds = stage + (size_t)(st->geo.threads / 64) * 512 * st->max_bits;
  }
  const rsq_status s = launch(fn, st, a, stream, start_event, stop_event, lds);
  if (s != RSQ_OK) return s;
  st->t += 1;
  if (st->bypass) st->n += 1;
  if (st->pw) st->n = std::min(st->n + 1, st->pw);
  return RSQ_OK;
}

}  // namespace

extern "C" {

rsq_status rsq_decode_step_timed(rsq_state* st, const void* q, const void* k, const void* v, const float* alpha,
                                 const float* beta, float* o, void* stream, void* start_event, void* stop_event) {
  return decode_step(st, q, k, v, alpha, beta, o, stream, start_event, stop_event, nullptr);
}

rsq_status rsq_decode_step_diag(rsq_state* st, const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, float* o, float* acc, float* ratio, uint32_t* counts,
                                void* stream) {
  const DiagBuffers dg{acc, ratio, counts};
  return decode_step(st, q, k, v, alpha, beta, o, stream, nullptr, nullptr, &dg);
}

rsq_status rsq_merge_bypass_timed(rsq_state* st, void* stream, void* start_event, void* stop_event) {
  if (!st) return fail(RSQ_E_INVALID, "state is NULL");
  if (!st->bypass) return fail(RSQ_E_NO_BYPASS, "this state has no low-rank bypass");
  {
    const rsq_status cs = refuse_capture(stream, "a bypass merge");
    if (cs != RSQ_OK) return cs;
  }
  StepArgs a = base_args(st);
  a.t_next = st->t;
  rsq::DecodeFn fn = rsq::merge_kernel_for(st->geo.cl);
  if (!fn) return fail(RSQ_E_UNSUPPORTED, "no merge kernel for this configuration");
  const rsq_status s = launch(fn, st, a, stream, start_event, stop_event, st->geo.lds_merge);
  if (s != RSQ_OK) return s;
  st->n = st->cfg.lrb_k;
  return RSQ_OK;
}

rsq_status rsq_merge_bypass(rsq_state* st, void* stream) {
  return rsq_merge_bypass_timed(st, stream, nullptr, nullptr);
}

rsq_status rsq_readout(const rsq_state* st, const void* q, float* o, void* stream) {
  if (!st) return fail(RSQ_E_INVALID, "state is NULL");
  if (!q || !o) return fail(RSQ_E_INVALID, "q and o must be non-NULL");
  if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(o) % 16)
    return fail(RSQ_E_INVALID, "q and o must be 16-byte aligned");
  StepArgs a = base_args(const_cast<rsq_state*>(st));
  a.q = q;
  a.o = o;
  rsq::DecodeFn fn = rsq::readout_kernel_for(st->geo.cl);
  return launch(fn, st, a, stream);
}

rsq_status rsq_get_status(rsq_state* st, uint32_t* flags, void* stream) {
  if (!st || !flags) return fail(RSQ_E_INVALID, "NULL argument");
  hipStream_t hs = (hipStream_t)stream;
  uint32_t* dev = reinterpret_cast<uint32_t*>(st->buf + st->layout.status);
  hipError_t e;
  if ((e = hipMemcpyAsync(flags, dev, 4, hipMemcpyDeviceToHost, hs)) != hipSuccess) return hip_fail(e, "status read");
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, hs, dev);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "status clear");
  if ((e = hipStreamSynchronize(hs)) != hipSuccess) return hip_fail(e, "stream sync");
  return RSQ_OK;
}

// Decay-aware per-head widths ("Low-Bit Recurrent States in Hybrid Language
// Models", abstract: distortion weights from the observability Gramian with
// normalised state ranges). Written out for the widths stored here:
//  * an error put into a state that decays by a_t per step keeps contributing
//    sum_t E[a^2]^t = 1 / (1 - E[a^2]) of its energy to later states;
//  * a b-bit symmetric step for range rho is rho / (2^(b-1) - 1), and the
//    rounding error energy scales with its square;
// so head h at width b costs w_h / (2^(b-1) - 1)^2, w_h = rho_h^2 / (1 - E[a_h^2]).
// Every upgrade (4->6, 6->8) costs 2 bits and a head's savings shrink as it
// widens (1/7^2 - 1/31^2 > 1/31^2 - 1/127^2), so taking upgrades largest
// saving first while the budget lasts minimises the total. Sorting all 2H
// upgrades by (saving desc, head asc, level asc) gives that order in
// O(H log H): a head's second upgrade never sorts before its first.
rsq_status rsq_allocate_head_bits(const float* decay_sq, const float* range, int32_t heads,
                                  float mean_bits, int32_t* bits_out) {
  if (!decay_sq || !range || !bits_out) return fail(RSQ_E_INVALID, "NULL argument");
  if (heads < 1 || heads > (1 << 20)) return fail(RSQ_E_INVALID, "heads = %d out of [1, 2^20]", heads);
  if (!(mean_bits >= 4.f && mean_bits <= 8.f)) return fail(RSQ_E_INVALID, "mean_bits must be in [4, 8]");
  struct Upgrade {
    double gain;
    int32_t head, level;
  };
  const double qsq[3] = {7.0 * 7.0, 31.0 * 31.0, 127.0 * 127.0};  // (2^(b-1) - 1)^2 for b = 4, 6, 8
  std::vector<Upgrade> ups;
  ups.reserve(2 * (size_t)heads);
  for (int32_t h = 0; h < heads; ++h) {
    const double d = decay_sq[h], r = range[h];
    if (!(d >= 0.0 && d < 1.0)) return fail(RSQ_E_INVALID, "decay_sq[%d] must be in [0, 1)", h);
    if (!(r >= 0.0 && std::isfinite(r))) return fail(RSQ_E_INVALID, "range[%d] must be finite and >= 0", h);
    const double w = (r * r) / (1.0 - d);
    for (int32_t l = 0; l < 2; ++l) {
      const double gain = w / qsq[l] - w / qsq[l + 1];
      if (gain > 0.0) ups.push_back({gain, h, l});
    }
  }
  std::sort(ups.begin(), ups.end(), [](const Upgrade& a, const Upgrade& b) {
    if (a.gain != b.gain) return a.gain > b.gain;
    if (a.head != b.head) return a.head < b.head;
    return a.level < b.level;
  });
  for (int32_t h = 0; h < heads; ++h) bits_out[h] = 4;
  const long budget = ((long)std::floor((double)mean_bits * (double)heads) - 4L * heads) / 2;
  const size_t take = std::min((size_t)budget, ups.size());
  for (size_t u = 0; u < take; ++u) bits_out[ups[u].head] += 2;
  return RSQ_OK;
}

}  // extern "C"
