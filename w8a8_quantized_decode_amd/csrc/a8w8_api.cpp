// C-ABI layer of liba8w8: argument validation, workspace carving and kernel launches.
//
// Every check runs on the host before anything is enqueued (the pages' serving path
// validates its configuration before execution, pypto-serving PR #48, commit "support
// A8W8 online serving"; and the down-projection tiling is guarded against silent
// truncation, pypto-lib PR #810, CodeRabbit nitpick on the down-projection constants).
//
// Launch chains.  With at most kFuseMaxRows rows every GEMM quantizes its own input in
// its prologue, so a layer is four kernels (QKV, O, Gate/Up, Down) and the MLP block
// two (Gate/Up, Down).  With more rows the per-row statistics would be re-derived by
// too many workgroups, so separate row-quantization kernels run before each GEMM.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/a8w8.h"
#include "attention_args.h"
#include "internal.h"

using namespace a8w8;

namespace {

constexpr int64_t kMaxK = 131072;  // 128 * 127 * K stays below 2^31
// The stream-K GEMM runs one grid row per 64 activation rows, and a grid dimension holds
// at most 65535 of them.
constexpr int64_t kMaxM = int64_t(65535) * 64;
constexpr size_t kAlign = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Linear carving of a workspace; with base == nullptr it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = round_up(off, kAlign);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  size_t size() const { return round_up(off, kAlign); }
};

// Every workspace layout starts with the two tag words of the decode GEMMs, so no
// other use of the workspace overwrites them between decode calls.
uint32_t* take_epoch(Carver& c) { return c.take<uint32_t>(2); }

bool valid_split(int s) { return s == 1 || s == 2 || s == 4 || s == 8; }

// Records the caller's timing events around the kernel with role `kernel`.
struct Timer {
  hipEvent_t start = nullptr, stop = nullptr;
  int kernel = -1;
  hipStream_t stream;
  Timer(const a8w8_mlp_taps* t, hipStream_t st)
      : start(t ? static_cast<hipEvent_t>(t->ev_start) : nullptr),
        stop(t ? static_cast<hipEvent_t>(t->ev_stop) : nullptr),
        kernel(t ? t->ev_kernel : -1),
        stream(st) {}
  hipError_t before(int k) const {
    return (start && stop && k == kernel) ? hipEventRecord(start, stream) : hipSuccess;
  }
  hipError_t after(int k) const {
    return (start && stop && k == kernel) ? hipEventRecord(stop, stream) : hipSuccess;
  }
};

#define A8W8_HIP(call)                             \
  do {                                             \
    if ((call) != hipSuccess) return A8W8_ERR_HIP; \
  } while (0)

// ------------------------------------------------------------------ plans & workspace
struct ChainPlan {
  bool fused;
  StreamKPlan qkv, o, gu, dn;
};

ChainPlan plans_for(int64_t M, int64_t H, int64_t I, int64_t n_qkv, int split_k, bool layer,
                    bool fused) {
  ChainPlan c{};
  c.fused = fused;
  if (layer) {
    c.qkv = plan_streamk(EPI_BF16, M, n_qkv, H, 1, fused);
    c.o = plan_streamk(EPI_BF16_RES, M, H, H, 1, fused);
  }
  c.gu = plan_streamk(EPI_SILU, M, I, H, 1, fused);
  c.dn = plan_streamk(EPI_DOWN, M, H, I, split_k, fused);
  return c;
}

// Every GEMM quantizes its own input in its prologue when the rows are few and each
// plan fits the prologue's LDS and register budget; otherwise row-quantization kernels
// run before the GEMMs.
ChainPlan make_plan(int64_t M, int64_t H, int64_t I, int64_t n_qkv, int split_k, bool layer) {
  ChainPlan c = plans_for(M, H, I, n_qkv, split_k, layer, true);
  bool ok = M <= kFuseMaxRows && streamk_fusable(c.gu, M, H, true) &&
            streamk_fusable(c.dn, M, I, false);
  if (layer) ok = ok && streamk_fusable(c.qkv, M, H, true) && streamk_fusable(c.o, M, H, true);
  return ok ? c : plans_for(M, H, I, n_qkv, split_k, layer, false);
}

// True when the GEMM reads its given codes from global memory in the 16-row tiled order
// (the row-quantization kernel before it then writes them so).
bool codes_tiled(const StreamKPlan& p) { return p.use_decode && p.dec.gcodes; }

// Rows of a codes buffer: the tiled order always holds 16.
size_t code_rows(int64_t M) { return size_t(M < 16 ? 16 : M); }

// Layout: done words and tagged partial-sum slots, shared by the GEMMs (they run one
// after another on the stream; done words and slot tags carry the GEMM's number), then
// the intermediate activations.
struct Buffers {
  uint32_t* epoch;          // [2] tag words, alternately read and advanced by the GEMMs
  int32_t* slots;
  uint64_t* dones;
  int8_t* q_in;
  float* s_in;
  uint16_t* qkv;
  int8_t* q_a;
  float* s_a;
  uint16_t* h1;
  int8_t* q_x;
  float* s_x;
  float* h;
  float* pmax;
  int8_t* q_h;
  float* s_h;
};

Buffers carve(Carver& c, const ChainPlan& pl, int64_t M, int64_t H, int64_t I, int64_t n_qkv,
              bool layer) {
  Buffers b{};
  size_t slot_elems = pl.gu.slot_elems;
  size_t done_elems = pl.gu.done_elems;
  auto widen = [&](const StreamKPlan& q) {
    if (q.slot_elems > slot_elems) slot_elems = q.slot_elems;
    if (q.done_elems > done_elems) done_elems = q.done_elems;
  };
  widen(pl.dn);
  if (layer) {
    widen(pl.qkv);
    widen(pl.o);
  }
  b.epoch = take_epoch(c);
  b.dones = c.take<uint64_t>(done_elems);
  b.slots = c.take<int32_t>(slot_elems);
  if (layer) {
    if (!pl.fused) {
      b.q_in = c.take<int8_t>(code_rows(M) * H);
      b.s_in = c.take<float>(size_t(M));
      b.q_a = c.take<int8_t>(code_rows(M) * H);
      b.s_a = c.take<float>(size_t(M));
    }
    b.qkv = c.take<uint16_t>(size_t(M) * n_qkv);
    b.h1 = c.take<uint16_t>(size_t(M) * H);
  }
  if (!pl.fused) {
    b.q_x = c.take<int8_t>(code_rows(M) * H);
    b.s_x = c.take<float>(size_t(M));
    b.q_h = c.take<int8_t>(code_rows(M) * I);
    b.s_h = c.take<float>(size_t(M));
  }
  b.h = c.take<float>(size_t(M) * I);
  b.pmax = c.take<float>(size_t(I / 16) * M);
  return b;
}

a8w8_status check_mlp_shapes(int64_t M, int64_t H, int64_t I, int split_k) {
  if (M < 0 || H <= 0 || I <= 0) return A8W8_ERR_SHAPE;
  if (!valid_split(split_k)) return A8W8_ERR_SHAPE;
  if (H % 64 || I % (64 * int64_t(split_k))) return A8W8_ERR_SHAPE;
  if (H > kMaxK || I > kMaxK) return A8W8_ERR_SHAPE;
  if (M > kMaxM) return A8W8_ERR_SHAPE;
  return A8W8_OK;
}

a8w8_status check_qweight(const a8w8_qweight& w) {
  if (!w.w || !w.scale) return A8W8_ERR_NULL;
  if (w.layout != A8W8_LAYOUT_ROWMAJOR && w.layout != A8W8_LAYOUT_TILED) return A8W8_ERR_SHAPE;
  if (!aligned16(w.w) || !aligned16(w.scale)) return A8W8_ERR_ALIGN;
  return A8W8_OK;
}

int layout_of(const a8w8_qweight& w) {
  return w.layout == A8W8_LAYOUT_TILED ? LAYOUT_TILED : LAYOUT_ROWMAJOR;
}

// GEMM number g of a call (calls run an even number of them) reads tag word g % 2 and
// advances the other one.
StreamKArgs gemm_args(int epi, const StreamKPlan& pl, int64_t M, int64_t N, int64_t K,
                      const a8w8_qweight& w, const Buffers& b, int g_in_call) {
  StreamKArgs g{};
  g.epi = epi;
  g.layout = layout_of(w);
  g.M = M;
  g.N = N;
  g.K = K;
  g.parts = 1;
  g.g = pl.geom;
  g.g2 = pl.geom2;
  g.wgs1 = pl.wgs1;
  g.toff2 = pl.toff2;
  g.act_row = pl.act_row;
  g.epoch_in = b.epoch + (g_in_call & 1);
  g.epoch_out = b.epoch + ((g_in_call + 1) & 1);
  g.w0 = w.w;
  g.sw0 = w.scale;
  g.slots = b.slots;
  g.dones = b.dones;
  return g;
}

// ------------------------------------------------------------------ prefill (W8A16)
struct PrefillBuffers {
  uint16_t* a;       // BF16 activations rne_bf16(RMSNorm(x)), prefill operand layout
  uint16_t* h;       // BF16 silu(g) * u, prefill operand layout
  float* slots;      // partial sums of split tiles
  uint16_t* qkv;     // layer: [M, n_qkv] BF16 QKV projection
  uint16_t* h1;      // layer: [M, H] BF16 attention-block output
};

// n_qkv > 0: the layer (QKV and O GEMMs before the MLP, their outputs kept here).
PrefillBuffers carve_prefill(Carver& c, int64_t M, int64_t H, int64_t I, int64_t n_qkv = 0) {
  const PrefillPlan gu = plan_prefill(EPI_PF_SILU, M, I, H);
  const PrefillPlan dn = plan_prefill(EPI_PF_RES, M, H, I);
  int64_t grid = gu.grid > dn.grid ? gu.grid : dn.grid;
  if (n_qkv > 0) {
    const PrefillPlan q = plan_prefill(EPI_PF_RES, M, n_qkv, H);
    const PrefillPlan o = plan_prefill(EPI_PF_RES, M, H, H);
    if (q.grid > grid) grid = q.grid;
    if (o.grid > grid) grid = o.grid;
  }
  const int64_t Mp = (M + 31) / 32 * 32;  // the operand layout pads rows to 32
  PrefillBuffers b{};
  take_epoch(c);
  b.a = c.take<uint16_t>(size_t(Mp) * H);
  b.h = c.take<uint16_t>(size_t(Mp) * I);
  b.slots = c.take<float>(size_t(2 * grid) * prefill_slot_floats());
  if (n_qkv > 0) {
    b.qkv = c.take<uint16_t>(size_t(M) * n_qkv);
    b.h1 = c.take<uint16_t>(size_t(M) * H);
  }
  return b;
}

bool prefill_shapes_ok(int64_t M, int64_t H, int64_t I) {
  return I % prefill_tile_channels(EPI_PF_SILU) == 0 &&
         H % prefill_tile_channels(EPI_PF_RES) == 0 && H % 256 == 0 && I % 256 == 0 &&
         M * (H > I ? H : I) < (int64_t(1) << 31);
}

a8w8_status run_mlp_prefill(const uint16_t* x, const uint16_t* gamma, float eps,
                            const a8w8_qweight& gate, const a8w8_qweight& up,
                            const a8w8_qweight& down, const uint16_t* res, uint16_t* out,
                            int64_t M, int64_t H, int64_t I, const PrefillBuffers& b,
                            const a8w8_mlp_taps* t, const Timer& tm, hipStream_t st) {
  // RMSNorm, narrowed to BF16 (the MFMA operand type).
  QuantRowsArgs q{};
  q.x = x;
  q.ldx = H;
  q.gamma = gamma;
  q.eps = eps;
  q.M = M;
  q.K = H;
  q.xn_tap = t ? t->xn : nullptr;
  q.a_bf16 = b.a;
  q.a_bf16_tiled = 1;
  q.a_bf16_tap = t ? t->a_bf16 : nullptr;
  q.write_codes = 0;
  A8W8_HIP(tm.before(A8W8_KERNEL_QUANT_POST));
  A8W8_HIP(launch_quant_rows(q, st));
  A8W8_HIP(tm.after(A8W8_KERNEL_QUANT_POST));

  // Gate/Up on BF16-dequantized weight tiles, FP32 accumulate, h = rne_bf16(silu(g) * u).
  PrefillGemmArgs g{};
  g.epi = EPI_PF_SILU;
  g.layout = layout_of(gate);
  g.M = M;
  g.N = I;
  g.K = H;
  g.act = b.a;
  g.w0 = gate.w;
  g.sw0 = gate.scale;
  g.w1 = up.w;
  g.sw1 = up.scale;
  g.out = b.h;
  g.tap_h = t ? t->h_bf16 : nullptr;
  g.tap_g = t ? t->g : nullptr;
  g.tap_u = t ? t->u : nullptr;
  g.slots = b.slots;
  A8W8_HIP(tm.before(A8W8_KERNEL_GATE_UP));
  A8W8_HIP(launch_prefill_gemm(g, st));
  A8W8_HIP(tm.after(A8W8_KERNEL_GATE_UP));

  // Down, FP32 accumulate, out = rne_bf16(d + res) in the same kernel.
  PrefillGemmArgs d{};
  d.epi = EPI_PF_RES;
  d.layout = layout_of(down);
  d.M = M;
  d.N = H;
  d.K = I;
  d.act = b.h;
  d.w0 = down.w;
  d.sw0 = down.scale;
  d.out = out;
  d.ldo = H;
  d.res = res;
  d.ldr = H;
  d.tap_d = t ? t->d : nullptr;
  d.slots = b.slots;
  A8W8_HIP(tm.before(A8W8_KERNEL_DOWN));
  A8W8_HIP(launch_prefill_gemm(d, st));
  A8W8_HIP(tm.after(A8W8_KERNEL_DOWN));
  return A8W8_OK;
}

// tiled: the codes in the 16-row tiled order a decode GEMM reads from global memory.
hipError_t quant_kernel(const void* x, int64_t ldx, int f32, const uint16_t* gamma, float eps,
                        int64_t M, int64_t K, int8_t* q, float* s, float* xn_tap, int8_t* q_tap,
                        float* s_tap, hipStream_t st, bool tiled = false) {
  QuantRowsArgs a{};
  a.q_tiled = tiled ? 1 : 0;
  a.x = x;
  a.ldx = ldx;
  a.x_is_f32 = f32;
  a.gamma = gamma;
  a.eps = eps;
  a.M = M;
  a.K = K;
  a.q = q;
  a.s = s;
  a.xn_tap = xn_tap;
  a.q_tap = q_tap;
  a.s_tap = s_tap;
  a.write_codes = 1;
  return launch_quant_rows(a, st);
}

// Enqueues the decode MLP chain (Gate/Up, then Down) as GEMMs g0 and g0 + 1 of the call.
a8w8_status run_mlp_decode(const uint16_t* x, const uint16_t* gamma, float eps,
                           const a8w8_qweight& gate, const a8w8_qweight& up,
                           const a8w8_qweight& down, const uint16_t* res, uint16_t* out,
                           int64_t M, int64_t H, int64_t I, int split_k, const ChainPlan& pl,
                           const Buffers& b, int g0, const a8w8_mlp_taps* t,
                           const Timer& tm, hipStream_t st) {
  // Gate/Up GEMM (input RMSNorm + quantization fused or separate), SiLU(g) * u -> h.
  StreamKArgs g = gemm_args(EPI_SILU, pl.gu, M, I, H, gate, b, g0);
  g.w1 = up.w;
  g.sw1 = up.scale;
  g.h = b.h;
  g.ldh = I;
  g.pmax_out = b.pmax;
  g.tap_acc0 = t ? t->acc_gate : nullptr;
  g.tap_acc1 = t ? t->acc_up : nullptr;
  g.tap_h = t ? t->h : nullptr;
  if (pl.fused) {
    g.prologue = PRO_QUANT_BF16;
    g.x = x;
    g.ldx = H;
    g.gamma = gamma;
    g.eps = eps;
    g.tap_xn = t ? t->xn : nullptr;
    g.tap_q = t ? t->q_x : nullptr;
    g.tap_s = t ? t->s_x : nullptr;
  } else {
    A8W8_HIP(tm.before(A8W8_KERNEL_QUANT_POST));
    A8W8_HIP(quant_kernel(x, H, 0, gamma, eps, M, H, b.q_x, b.s_x, t ? t->xn : nullptr,
                          t ? t->q_x : nullptr, t ? t->s_x : nullptr, st, codes_tiled(pl.gu)));
    A8W8_HIP(tm.after(A8W8_KERNEL_QUANT_POST));
    g.prologue = PRO_CODES;
    g.a = b.q_x;
    g.lda = H;
    g.sa = b.s_x;
  }
  A8W8_HIP(tm.before(A8W8_KERNEL_GATE_UP));
  A8W8_HIP(launch_streamk(g, pl.gu, st));
  A8W8_HIP(tm.after(A8W8_KERNEL_GATE_UP));

  // Down: per-row requantization of h, split-K partials, + residual, RNE to BF16.
  StreamKArgs d = gemm_args(EPI_DOWN, pl.dn, M, H, I, down, b, g0 + 1);
  d.parts = split_k;
  d.out = out;
  d.ldo = H;
  d.res = res;
  d.ldr = H;
  d.tap_acc0 = t ? t->acc_down : nullptr;
  d.tap_p = t ? t->p_down : nullptr;
  d.once = out == res ? 1 : 0;
  if (pl.fused) {
    d.prologue = PRO_REQUANT_F32;
    d.hin = b.h;
    d.ldhin = I;
    d.pmax = b.pmax;
    d.npmax = I / 16;
    d.tap_q = t ? t->q_h : nullptr;
    d.tap_s = t ? t->s_h : nullptr;
  } else {
    // The row scales come from the Gate/Up epilogue's partial maxima of h.
    A8W8_HIP(tm.before(A8W8_KERNEL_REQUANT));
    QuantRowsArgs rq{};
    rq.x = b.h;
    rq.ldx = I;
    rq.x_is_f32 = 1;
    rq.M = M;
    rq.K = I;
    rq.q = b.q_h;
    rq.q_tiled = codes_tiled(pl.dn) ? 1 : 0;
    rq.s = b.s_h;
    rq.q_tap = t ? t->q_h : nullptr;
    rq.s_tap = t ? t->s_h : nullptr;
    rq.write_codes = 1;
    rq.pmax = b.pmax;
    rq.npmax = I / 16;
    A8W8_HIP(M <= 65535 ? launch_requant_pmax(rq, st) : launch_quant_rows(rq, st));
    A8W8_HIP(tm.after(A8W8_KERNEL_REQUANT));
    d.prologue = PRO_CODES;
    d.a = b.q_h;
    d.lda = I;
    d.sa = b.s_h;
  }
  A8W8_HIP(tm.before(A8W8_KERNEL_DOWN));
  A8W8_HIP(launch_streamk(d, pl.dn, st));
  A8W8_HIP(tm.after(A8W8_KERNEL_DOWN));
  return A8W8_OK;
}

}  // namespace

extern "C" {

const char* a8w8_status_string(a8w8_status s) {
  switch (s) {
    case A8W8_OK: return "A8W8_OK";
    case A8W8_ERR_NULL: return "A8W8_ERR_NULL: a required pointer is NULL";
    case A8W8_ERR_SHAPE: return "A8W8_ERR_SHAPE: unsupported or inconsistent sizes";
    case A8W8_ERR_ALIGN: return "A8W8_ERR_ALIGN: a pointer is not 16-byte aligned";
    case A8W8_ERR_WORKSPACE: return "A8W8_ERR_WORKSPACE: workspace missing or too small";
    case A8W8_ERR_UNSUPPORTED: return "A8W8_ERR_UNSUPPORTED: not implemented in this build";
    case A8W8_ERR_HIP: return "A8W8_ERR_HIP: a HIP call or kernel launch failed";
  }
  return "A8W8_ERR_UNKNOWN";
}

int a8w8_version(void) { return 300; }

a8w8_status a8w8_pack_weight(const int8_t* w, int64_t N, int64_t K, int8_t* w_tiled,
                             void* stream) {
  if (N <= 0 || K <= 0 || N % 16 || K % 64) return A8W8_ERR_SHAPE;
  if (!w || !w_tiled) return A8W8_ERR_NULL;
  if (!aligned16(w) || !aligned16(w_tiled)) return A8W8_ERR_ALIGN;
  A8W8_HIP(launch_pack_tiled(w, N, K, w_tiled, static_cast<hipStream_t>(stream)));
  return A8W8_OK;
}

a8w8_status a8w8_quantize_rows(const uint16_t* x_bf16, int64_t ldx, const uint16_t* gamma_bf16,
                               float eps, int64_t M, int64_t K, int8_t* q_out,
                               float* row_scale_out, float* xn_tap, void* stream) {
  if (M < 0 || K <= 0 || K % 8 || ldx < K || ldx % 8 || M > (int64_t(1) << 31) - 1)
    return A8W8_ERR_SHAPE;
  if (M == 0) return A8W8_OK;
  if (!x_bf16 || !q_out || !row_scale_out) return A8W8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(q_out) || !aligned16(row_scale_out) ||
      (gamma_bf16 && !aligned16(gamma_bf16)) || (xn_tap && !aligned16(xn_tap)))
    return A8W8_ERR_ALIGN;
  A8W8_HIP(quant_kernel(x_bf16, ldx, 0, gamma_bf16, eps, M, K, q_out, row_scale_out, xn_tap,
                        nullptr, nullptr, static_cast<hipStream_t>(stream)));
  return A8W8_OK;
}

a8w8_status a8w8_linear(const int8_t* q, const float* row_scale, a8w8_qweight W,
                        const uint16_t* residual_bf16, int64_t M, int64_t N, int64_t K,
                        uint16_t* y_bf16, int32_t* acc_i32_tap, void* stream) {
  if (M < 0 || N <= 0 || K <= 0 || K % 64 || N % 16 || K > kMaxK || M > kMaxM)
    return A8W8_ERR_SHAPE;
  if (M == 0) return A8W8_OK;
  if (!q || !row_scale || !y_bf16) return A8W8_ERR_NULL;
  if (a8w8_status s = check_qweight(W)) return s;
  if (!aligned16(q) || !aligned16(row_scale) || !aligned16(y_bf16) ||
      (residual_bf16 && !aligned16(residual_bf16)) || (acc_i32_tap && !aligned16(acc_i32_tap)))
    return A8W8_ERR_ALIGN;
  LinearArgs g{};
  g.epi = residual_bf16 ? EPI_BF16_RES : EPI_BF16;
  g.layout = layout_of(W);
  g.M = M;
  g.N = N;
  g.K = K;
  g.a = q;
  g.lda = K;
  g.sa = row_scale;
  g.w0 = W.w;
  g.sw0 = W.scale;
  g.out = y_bf16;
  g.ldo = N;
  g.res = residual_bf16;
  g.ldr = N;
  g.tap_acc0 = acc_i32_tap;
  A8W8_HIP(launch_linear(g, static_cast<hipStream_t>(stream)));
  return A8W8_OK;
}

size_t a8w8_workspace_bytes(int op, int64_t M, int64_t H, int64_t I, int64_t n_qkv,
                            int split_k, int mode) {
  if (check_mlp_shapes(M, H, I, split_k) != A8W8_OK) return 0;
  if (mode == A8W8_MODE_PREFILL_W8A16) {
    if (!prefill_shapes_ok(M, H, I)) return 0;
    Carver c(nullptr);
    if (op == A8W8_OP_MLP_BLOCK) {
      carve_prefill(c, M, H, I);
    } else if (op == A8W8_OP_LAYER_LINEARS) {
      if (n_qkv <= 0 || n_qkv % prefill_tile_channels(EPI_PF_RES)) return 0;
      carve_prefill(c, M, H, I, n_qkv);
    } else {
      return 0;
    }
    return c.size() > 0 ? c.size() : kAlign;
  }
  if (mode != A8W8_MODE_DECODE_A8W8) return 0;
  bool layer;
  if (op == A8W8_OP_MLP_BLOCK) {
    layer = false;
    n_qkv = 0;
  } else if (op == A8W8_OP_LAYER_LINEARS) {
    if (n_qkv <= 0 || n_qkv % 16) return 0;
    layer = true;
  } else {
    return 0;
  }
  const ChainPlan pl = make_plan(M, H, I, n_qkv, split_k, layer);
  Carver c(nullptr);
  carve(c, pl, M, H, I, n_qkv, layer);
  return c.size() > 0 ? c.size() : kAlign;
}

a8w8_status a8w8_mlp_block(const uint16_t* x_bf16, const uint16_t* gamma_bf16, float eps,
                           a8w8_qweight gate, a8w8_qweight up, a8w8_qweight down,
                           const uint16_t* residual_bf16, uint16_t* out_bf16, int64_t M,
                           int64_t H, int64_t I, int split_k, int mode, void* workspace,
                           size_t ws_bytes, const a8w8_mlp_taps* taps, void* stream) {
  if (a8w8_status s = check_mlp_shapes(M, H, I, split_k)) return s;
  if (mode != A8W8_MODE_DECODE_A8W8 && mode != A8W8_MODE_PREFILL_W8A16) return A8W8_ERR_SHAPE;
  if (M == 0) return A8W8_OK;
  if (!x_bf16 || !gamma_bf16 || !residual_bf16 || !out_bf16) return A8W8_ERR_NULL;
  for (const a8w8_qweight* w : {&gate, &up, &down})
    if (a8w8_status s = check_qweight(*w)) return s;
  if (!aligned16(x_bf16) || !aligned16(gamma_bf16) || !aligned16(residual_bf16) ||
      !aligned16(out_bf16))
    return A8W8_ERR_ALIGN;
  if (mode == A8W8_MODE_PREFILL_W8A16 && !prefill_shapes_ok(M, H, I)) return A8W8_ERR_SHAPE;
  const size_t need = a8w8_workspace_bytes(A8W8_OP_MLP_BLOCK, M, H, I, 0, split_k, mode);
  if (!workspace || ws_bytes < need) return A8W8_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return A8W8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Timer tm(taps, st);
  if (mode == A8W8_MODE_PREFILL_W8A16) {
    Carver c(workspace);
    const PrefillBuffers pb = carve_prefill(c, M, H, I);
    return run_mlp_prefill(x_bf16, gamma_bf16, eps, gate, up, down, residual_bf16, out_bf16, M,
                           H, I, pb, taps, tm, st);
  }
  const ChainPlan pl = make_plan(M, H, I, 0, split_k, false);
  Carver c(workspace);
  const Buffers b = carve(c, pl, M, H, I, 0, false);
  return run_mlp_decode(x_bf16, gamma_bf16, eps, gate, up, down, residual_bf16, out_bf16, M, H,
                        I, split_k, pl, b, 0, taps, tm, st);
}

static a8w8_status make_qk_args(const uint16_t*, int64_t, int, int, int, const uint16_t*,
                                const uint16_t*, float, const float*, const float*, int64_t,
                                const int32_t*, const int32_t*, int64_t, uint16_t*, uint16_t*,
                                int64_t, int64_t, uint16_t*, QkRopeArgs&);
static a8w8_status make_attn_args(const uint16_t*, int64_t, int, int, int, const uint16_t*,
                                  const uint16_t*, int64_t, int64_t, const int32_t*, int64_t,
                                  const int32_t*, float, uint16_t*, void*, size_t, AttnArgs&);

// The decode layer: QKV, then either the identity attention on the Q slice (att ==
// nullptr) or QK-norm + RoPE + KV write and decode attention, then O (+ x) and the MLP.
// ------------------------------------------------------------------ allocation-free entry
// Workspace of a8w8_layer_linears_static: a file-scope device array, one copy per GPU, held
// until the process ends.  Host code never passes the array's name to a kernel (on the
// host it only stands for the symbol); the device address of each GPU's copy is looked up
// once per device and kept here.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`; A8W8_ERR_HIP if it cannot be resolved.
a8w8_status static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return A8W8_ERR_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return A8W8_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return A8W8_OK;
}

static a8w8_status layer_decode(const uint16_t* x_bf16, const uint16_t* gamma_in_bf16,
                                const uint16_t* gamma_post_bf16, float eps, a8w8_qweight qkv,
                                a8w8_qweight o, a8w8_qweight gate, a8w8_qweight up,
                                a8w8_qweight down, int64_t M, int64_t H, int64_t I,
                                int n_q_heads, int n_kv_heads, int head_dim, int split_k,
                                const a8w8_attention_step* att, uint16_t* qkv_out_bf16,
                                uint16_t* h1_out_bf16, uint16_t* out_bf16, void* workspace,
                                size_t ws_bytes, const a8w8_layer_taps* taps, void* stream,
                                bool static_ws = false) {
  if (a8w8_status s = check_mlp_shapes(M, H, I, split_k)) return s;
  if (n_q_heads <= 0 || n_kv_heads < 0 || head_dim <= 0) return A8W8_ERR_SHAPE;
  if (int64_t(n_q_heads) * head_dim != H) return A8W8_ERR_SHAPE;
  const int64_t n_qkv = (int64_t(n_q_heads) + 2 * int64_t(n_kv_heads)) * head_dim;
  if (n_qkv % 16) return A8W8_ERR_SHAPE;
  if (M == 0) return A8W8_OK;
  if (!x_bf16 || !gamma_in_bf16 || !gamma_post_bf16 || !out_bf16) return A8W8_ERR_NULL;
  for (const a8w8_qweight* w : {&qkv, &o, &gate, &up, &down})
    if (a8w8_status s = check_qweight(*w)) return s;
  if (!aligned16(x_bf16) || !aligned16(gamma_in_bf16) || !aligned16(gamma_post_bf16) ||
      !aligned16(out_bf16) || (qkv_out_bf16 && !aligned16(qkv_out_bf16)) ||
      (h1_out_bf16 && !aligned16(h1_out_bf16)))
    return A8W8_ERR_ALIGN;
  const size_t need = a8w8_workspace_bytes(A8W8_OP_LAYER_LINEARS, M, H, I, n_qkv, split_k,
                                           A8W8_MODE_DECODE_A8W8);
  if (static_ws) {
    // The library's own workspace: checked against its size, then looked up (the first
    // call on a device resolves that device's copy).
    if (need > kStaticScratchBytes) return A8W8_ERR_WORKSPACE;
    if (a8w8_status e = static_scratch(&workspace)) return e;
    ws_bytes = kStaticScratchBytes;
  }
  if (!workspace || ws_bytes < need) return A8W8_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return A8W8_ERR_ALIGN;
  const ChainPlan pl = make_plan(M, H, I, n_qkv, split_k, true);
  Carver c(workspace);
  const Buffers b = carve(c, pl, M, H, I, n_qkv, true);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const a8w8_mlp_taps* mt = taps ? &taps->mlp : nullptr;
  const Timer tm(mt, st);
  uint16_t* qkv_buf = qkv_out_bf16 ? qkv_out_bf16 : b.qkv;
  uint16_t* h1 = h1_out_bf16 ? h1_out_bf16 : b.h1;
  // Attention arguments are checked before anything is enqueued.
  QkRopeArgs qa{};
  AttnArgs aa{};
  if (att) {
    if (!att->q_rot_bf16 || !att->attn_bf16) return A8W8_ERR_NULL;
    if (a8w8_status e = make_qk_args(qkv_buf, M, n_q_heads, n_kv_heads, head_dim,
                                     att->q_gamma_bf16, att->k_gamma_bf16, att->qk_eps,
                                     att->cos_table, att->sin_table, att->max_pos,
                                     att->positions, att->block_table, att->blocks_per_seq,
                                     att->k_cache_bf16, att->v_cache_bf16, att->num_blocks,
                                     att->block_size, att->q_rot_bf16, qa))
      return e;
    if (a8w8_status e = make_attn_args(att->q_rot_bf16, M, n_q_heads, n_kv_heads, head_dim,
                                       att->k_cache_bf16, att->v_cache_bf16, att->num_blocks,
                                       att->block_size, att->block_table, att->blocks_per_seq,
                                       att->context_lens, att->scale, att->attn_bf16,
                                       att->attn_workspace, att->attn_ws_bytes, aa))
      return e;
  }
  // O's input rows: the attention output, or the Q slice of QKV (identity attention).
  const uint16_t* o_in = att ? att->attn_bf16 : qkv_buf;
  const int64_t o_ld = att ? H : n_qkv;


  // QKV projection (input RMSNorm + quantization fused or separate) -> BF16.
  StreamKArgs g = gemm_args(EPI_BF16, pl.qkv, M, n_qkv, H, qkv, b, 0);
  g.out = qkv_buf;
  g.ldo = n_qkv;
  g.tap_acc0 = taps ? taps->acc_qkv : nullptr;
  if (pl.fused) {
    g.prologue = PRO_QUANT_BF16;
    g.x = x_bf16;
    g.ldx = H;
    g.gamma = gamma_in_bf16;
    g.eps = eps;
    g.tap_xn = taps ? taps->xn_in : nullptr;
    g.tap_q = taps ? taps->q_in : nullptr;
    g.tap_s = taps ? taps->s_in : nullptr;
  } else {
    A8W8_HIP(tm.before(A8W8_KERNEL_QUANT_IN));
    A8W8_HIP(quant_kernel(x_bf16, H, 0, gamma_in_bf16, eps, M, H, b.q_in, b.s_in,
                          taps ? taps->xn_in : nullptr, taps ? taps->q_in : nullptr,
                          taps ? taps->s_in : nullptr, st, codes_tiled(pl.qkv)));
    A8W8_HIP(tm.after(A8W8_KERNEL_QUANT_IN));
    g.prologue = PRO_CODES;
    g.a = b.q_in;
    g.lda = H;
    g.sa = b.s_in;
  }
  A8W8_HIP(tm.before(A8W8_KERNEL_QKV));
  A8W8_HIP(launch_streamk(g, pl.qkv, st));
  A8W8_HIP(tm.after(A8W8_KERNEL_QKV));
  if (taps && taps->qkv)
    A8W8_HIP(hipMemcpyAsync(taps->qkv, qkv_buf, size_t(M) * n_qkv * sizeof(uint16_t),
                            hipMemcpyDeviceToDevice, st));

  if (att) {
    A8W8_HIP(launch_qk_rope(qa, st));
    A8W8_HIP(launch_decode_attention(aa, st));
  }

  // O's input rows are quantized and fed to O; O adds the layer input as residual -> h1.
  StreamKArgs og = gemm_args(EPI_BF16_RES, pl.o, M, H, H, o, b, 1);
  og.out = h1;
  og.ldo = H;
  og.res = x_bf16;
  og.ldr = H;
  og.tap_acc0 = taps ? taps->acc_o : nullptr;
  if (pl.fused) {
    og.prologue = PRO_QUANT_BF16;
    og.x = o_in;
    og.ldx = o_ld;
    og.tap_q = taps ? taps->q_attn : nullptr;
    og.tap_s = taps ? taps->s_attn : nullptr;
  } else {
    A8W8_HIP(tm.before(A8W8_KERNEL_QUANT_ATTN));
    A8W8_HIP(quant_kernel(o_in, o_ld, 0, nullptr, 0.0f, M, H, b.q_a, b.s_a, nullptr,
                          taps ? taps->q_attn : nullptr, taps ? taps->s_attn : nullptr, st,
                          codes_tiled(pl.o)));
    A8W8_HIP(tm.after(A8W8_KERNEL_QUANT_ATTN));
    og.prologue = PRO_CODES;
    og.a = b.q_a;
    og.lda = H;
    og.sa = b.s_a;
  }
  A8W8_HIP(tm.before(A8W8_KERNEL_O));
  A8W8_HIP(launch_streamk(og, pl.o, st));
  A8W8_HIP(tm.after(A8W8_KERNEL_O));
  if (taps && taps->h1)
    A8W8_HIP(hipMemcpyAsync(taps->h1, h1, size_t(M) * H * sizeof(uint16_t),
                            hipMemcpyDeviceToDevice, st));

  return run_mlp_decode(h1, gamma_post_bf16, eps, gate, up, down, h1, out_bf16, M, H, I,
                        split_k, pl, b, 2, mt, tm, st);
}

a8w8_status a8w8_layer_linears(const uint16_t* x_bf16, const uint16_t* gamma_in_bf16,
                               const uint16_t* gamma_post_bf16, float eps,
                               a8w8_qweight qkv, a8w8_qweight o, a8w8_qweight gate,
                               a8w8_qweight up, a8w8_qweight down, int64_t M, int64_t H,
                               int64_t I, int n_q_heads, int n_kv_heads, int head_dim,
                               int split_k, uint16_t* qkv_out_bf16, uint16_t* out_bf16,
                               void* workspace, size_t ws_bytes,
                               const a8w8_layer_taps* taps, void* stream) {
  return layer_decode(x_bf16, gamma_in_bf16, gamma_post_bf16, eps, qkv, o, gate, up, down, M,
                      H, I, n_q_heads, n_kv_heads, head_dim, split_k, nullptr, qkv_out_bf16,
                      nullptr, out_bf16, workspace, ws_bytes, taps, stream);
}

size_t a8w8_layer_linears_static_max_workspace(void) { return kStaticScratchBytes; }

a8w8_status a8w8_layer_linears_static(const uint16_t* x_bf16, const uint16_t* gamma_in_bf16,
                                      const uint16_t* gamma_post_bf16, float eps,
                                      a8w8_qweight qkv, a8w8_qweight o, a8w8_qweight gate,
                                      a8w8_qweight up, a8w8_qweight down, int64_t M, int64_t H,
                                      int64_t I, int n_q_heads, int n_kv_heads, int head_dim,
                                      int split_k, uint16_t* qkv_out_bf16, uint16_t* out_bf16,
                                      const a8w8_layer_taps* taps, void* stream) {
  return layer_decode(x_bf16, gamma_in_bf16, gamma_post_bf16, eps, qkv, o, gate, up, down, M,
                      H, I, n_q_heads, n_kv_heads, head_dim, split_k, nullptr, qkv_out_bf16,
                      nullptr, out_bf16, nullptr, 0, taps, stream, /*static_ws=*/true);
}

a8w8_status a8w8_decode_layer(const uint16_t* x_bf16, const uint16_t* gamma_in_bf16,
                              const uint16_t* gamma_post_bf16, float eps, a8w8_qweight qkv,
                              a8w8_qweight o, a8w8_qweight gate, a8w8_qweight up,
                              a8w8_qweight down, int64_t M, int64_t H, int64_t I,
                              int n_q_heads, int n_kv_heads, int head_dim, int split_k,
                              const a8w8_attention_step* attn, uint16_t* qkv_out_bf16,
                              uint16_t* h1_out_bf16, uint16_t* out_bf16, void* workspace,
                              size_t ws_bytes, void* stream) {
  if (!attn) return A8W8_ERR_NULL;
  return layer_decode(x_bf16, gamma_in_bf16, gamma_post_bf16, eps, qkv, o, gate, up, down, M,
                      H, I, n_q_heads, n_kv_heads, head_dim, split_k, attn, qkv_out_bf16,
                      h1_out_bf16, out_bf16, workspace, ws_bytes, nullptr, stream);
}

a8w8_status a8w8_layer_linears_prefill(const uint16_t* x_bf16, const uint16_t* gamma_in_bf16,
                                       const uint16_t* gamma_post_bf16, float eps,
                                       a8w8_qweight qkv, a8w8_qweight o, a8w8_qweight gate,
                                       a8w8_qweight up, a8w8_qweight down, int64_t M,
                                       int64_t H, int64_t I, int n_q_heads, int n_kv_heads,
                                       int head_dim, uint16_t* qkv_out_bf16,
                                       uint16_t* h1_out_bf16, uint16_t* out_bf16,
                                       void* workspace, size_t ws_bytes, void* stream) {
  if (a8w8_status s = check_mlp_shapes(M, H, I, 2)) return s;
  if (n_q_heads <= 0 || n_kv_heads < 0 || head_dim <= 0) return A8W8_ERR_SHAPE;
  if (int64_t(n_q_heads) * head_dim != H) return A8W8_ERR_SHAPE;
  const int64_t n_qkv = (int64_t(n_q_heads) + 2 * int64_t(n_kv_heads)) * head_dim;
  if (!prefill_shapes_ok(M, H, I) || n_qkv % prefill_tile_channels(EPI_PF_RES) ||
      M * n_qkv >= (int64_t(1) << 31))
    return A8W8_ERR_SHAPE;
  if (M == 0) return A8W8_OK;
  if (!x_bf16 || !gamma_in_bf16 || !gamma_post_bf16 || !out_bf16) return A8W8_ERR_NULL;
  for (const a8w8_qweight* w : {&qkv, &o, &gate, &up, &down})
    if (a8w8_status s = check_qweight(*w)) return s;
  if (!aligned16(x_bf16) || !aligned16(gamma_in_bf16) || !aligned16(gamma_post_bf16) ||
      !aligned16(out_bf16) || (qkv_out_bf16 && !aligned16(qkv_out_bf16)) ||
      (h1_out_bf16 && !aligned16(h1_out_bf16)))
    return A8W8_ERR_ALIGN;
  const size_t need = a8w8_workspace_bytes(A8W8_OP_LAYER_LINEARS, M, H, I, n_qkv, 2,
                                           A8W8_MODE_PREFILL_W8A16);
  if (!workspace || ws_bytes < need) return A8W8_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return A8W8_ERR_ALIGN;
  Carver c(workspace);
  const PrefillBuffers pb = carve_prefill(c, M, H, I, n_qkv);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Timer tm(nullptr, st);
  uint16_t* qkv_buf = qkv_out_bf16 ? qkv_out_bf16 : pb.qkv;
  uint16_t* h1_buf = h1_out_bf16 ? h1_out_bf16 : pb.h1;

  // a = rne_bf16(RMSNorm(x, gamma_in)) in the prefill operand layout.
  QuantRowsArgs q{};
  q.x = x_bf16;
  q.ldx = H;
  q.gamma = gamma_in_bf16;
  q.eps = eps;
  q.M = M;
  q.K = H;
  q.a_bf16 = pb.a;
  q.a_bf16_tiled = 1;
  q.write_codes = 0;
  A8W8_HIP(launch_quant_rows(q, st));
  // qkv = rne_bf16(a W'_qkv^T), row-major [M, n_qkv].
  PrefillGemmArgs g{};
  g.epi = EPI_PF_RES;
  g.layout = layout_of(qkv);
  g.M = M;
  g.N = n_qkv;
  g.K = H;
  g.act = pb.a;
  g.w0 = qkv.w;
  g.sw0 = qkv.scale;
  g.out = qkv_buf;
  g.ldo = n_qkv;
  g.res = nullptr;
  g.slots = pb.slots;
  A8W8_HIP(launch_prefill_gemm(g, st));
  // The Q slice (identity attention) into the operand layout: a BF16 copy.
  QuantRowsArgs qa{};
  qa.x = qkv_buf;
  qa.ldx = n_qkv;
  qa.M = M;
  qa.K = H;
  qa.a_bf16 = pb.a;
  qa.a_bf16_tiled = 1;
  qa.write_codes = 0;
  A8W8_HIP(launch_quant_rows(qa, st));
  // h1 = rne_bf16(attn W'_o^T + x).
  PrefillGemmArgs og{};
  og.epi = EPI_PF_RES;
  og.layout = layout_of(o);
  og.M = M;
  og.N = H;
  og.K = H;
  og.act = pb.a;
  og.w0 = o.w;
  og.sw0 = o.scale;
  og.out = h1_buf;
  og.ldo = H;
  og.res = x_bf16;
  og.ldr = H;
  og.slots = pb.slots;
  A8W8_HIP(launch_prefill_gemm(og, st));
  // The MLP block on h1, with h1 as its residual.
  return run_mlp_prefill(h1_buf, gamma_post_bf16, eps, gate, up, down, h1_buf, out_bf16, M, H,
                         I, pb, nullptr, tm, st);
}

// Validates the QK-norm + RoPE + KV step and fills its kernel arguments (a.M == 0 on
// return: nothing to launch).
static a8w8_status make_qk_args(const uint16_t* qkv_bf16, int64_t M, int n_q_heads,
                                int n_kv_heads, int head_dim, const uint16_t* q_gamma_bf16,
                                const uint16_t* k_gamma_bf16, float eps,
                                const float* cos_table, const float* sin_table,
                                int64_t max_pos, const int32_t* positions,
                                const int32_t* block_table, int64_t blocks_per_seq,
                                uint16_t* k_cache_bf16, uint16_t* v_cache_bf16,
                                int64_t num_blocks, int64_t block_size, uint16_t* q_out_bf16,
                                QkRopeArgs& a) {
  if (M < 0 || M > 65535 || n_q_heads <= 0 || n_kv_heads < 0 || head_dim <= 0 ||
      head_dim % 2 || head_dim > 512 || max_pos <= 0 || max_pos > (int64_t(1) << 31) - 1)
    return A8W8_ERR_SHAPE;
  if (n_q_heads + 2 * int64_t(n_kv_heads) > 65535) return A8W8_ERR_SHAPE;
  if (n_kv_heads > 0 && (blocks_per_seq <= 0 || num_blocks <= 0 || block_size <= 0 ||
                         num_blocks > (int64_t(1) << 31) - 1))
    return A8W8_ERR_SHAPE;
  if (M == 0) {
    a = QkRopeArgs{};
    return A8W8_OK;
  }
  if (!qkv_bf16 || !q_gamma_bf16 || !cos_table || !sin_table || !positions || !q_out_bf16)
    return A8W8_ERR_NULL;
  if (n_kv_heads > 0 && (!k_gamma_bf16 || !block_table || !k_cache_bf16 || !v_cache_bf16))
    return A8W8_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(cos_table) | reinterpret_cast<uintptr_t>(sin_table) |
       reinterpret_cast<uintptr_t>(positions) |
       reinterpret_cast<uintptr_t>(block_table)) & 3u)
    return A8W8_ERR_ALIGN;
  a = QkRopeArgs{};
  a.qkv = qkv_bf16;
  a.M = M;
  a.n_q = n_q_heads;
  a.n_kv = n_kv_heads;
  a.head_dim = head_dim;
  a.ld_qkv = (int64_t(n_q_heads) + 2 * int64_t(n_kv_heads)) * head_dim;
  a.q_gamma = q_gamma_bf16;
  a.k_gamma = k_gamma_bf16;
  a.eps = eps;
  a.cos_table = cos_table;
  a.sin_table = sin_table;
  a.max_pos = max_pos;
  a.positions = positions;
  a.block_table = block_table;
  a.blocks_per_seq = blocks_per_seq;
  a.k_cache = k_cache_bf16;
  a.v_cache = v_cache_bf16;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.q_out = q_out_bf16;
  a.ld_q = int64_t(n_q_heads) * head_dim;
  return A8W8_OK;
}

a8w8_status a8w8_qk_norm_rope_kv(const uint16_t* qkv_bf16, int64_t M, int n_q_heads,
                                 int n_kv_heads, int head_dim, const uint16_t* q_gamma_bf16,
                                 const uint16_t* k_gamma_bf16, float eps,
                                 const float* cos_table, const float* sin_table,
                                 int64_t max_pos, const int32_t* positions,
                                 const int32_t* block_table, int64_t blocks_per_seq,
                                 uint16_t* k_cache_bf16, uint16_t* v_cache_bf16,
                                 int64_t num_blocks, int64_t block_size, uint16_t* q_out_bf16,
                                 void* stream) {
  QkRopeArgs a;
  if (a8w8_status e = make_qk_args(qkv_bf16, M, n_q_heads, n_kv_heads, head_dim, q_gamma_bf16,
                                   k_gamma_bf16, eps, cos_table, sin_table, max_pos, positions,
                                   block_table, blocks_per_seq, k_cache_bf16, v_cache_bf16,
                                   num_blocks, block_size, q_out_bf16, a))
    return e;
  if (a.M == 0) return A8W8_OK;
  A8W8_HIP(launch_qk_rope(a, static_cast<hipStream_t>(stream)));
  return A8W8_OK;
}

// Small problems (at most kAttnWholeGroups (row, KV head) pairs of at most
// kAttnWholeChunks chunks of 64 positions) run one workgroup of eight waves per pair,
// each wave taking whole chunks, with no split and no merge.  Otherwise, positions per
// split: one workgroup per 64 positions while that keeps the grid under
// kAttnTargetGroups workgroups, otherwise whole multiples of 64 so that it does; grids of
// fewer than kAttnFourWaveChunks chunks run four waves per split.
constexpr int64_t kAttnWholeGroups = 64;
constexpr int64_t kAttnWholeChunks = 4;
constexpr int64_t kAttnTargetGroups = 2048;
constexpr int64_t kAttnFourWaveChunks = 512;
static bool attn_whole(int64_t M, int n_kv, int64_t max_ctx) {
  return M * n_kv <= kAttnWholeGroups && (max_ctx + 63) / 64 <= kAttnWholeChunks;
}
static int64_t attn_split_len(int64_t M, int n_kv, int64_t max_ctx) {
  const int64_t chunks = (max_ctx + 63) / 64;
  if (attn_whole(M, n_kv, max_ctx)) return chunks * 64;
  int64_t per = (M * n_kv * chunks + kAttnTargetGroups - 1) / kAttnTargetGroups;
  if (per < 1) per = 1;
  if (per > chunks) per = chunks;
  return per * 64;
}

static bool attn_shapes_ok(int64_t M, int n_q, int n_kv, int d, int64_t max_ctx) {
  return M >= 0 && M <= 65535 && n_kv > 0 && n_kv <= 65535 && n_q > 0 && n_q % n_kv == 0 &&
         n_q / n_kv <= 8 && (d == 64 || d == 128) && max_ctx > 0 &&
         max_ctx <= (int64_t(1) << 30);
}

size_t a8w8_decode_attention_workspace_bytes(int64_t M, int n_q_heads, int n_kv_heads,
                                             int head_dim, int64_t max_context) {
  if (!attn_shapes_ok(M, n_q_heads, n_kv_heads, head_dim, max_context)) return 0;
  const int64_t split = attn_split_len(M, n_kv_heads, max_context);
  const int64_t S = (max_context + split - 1) / split;
  if (S <= 1) return 0;
  int64_t n = 0;
  if (__builtin_mul_overflow(M * n_q_heads, S, &n) ||
      __builtin_mul_overflow(n, int64_t(head_dim + 2) * int64_t(sizeof(float)), &n))
    return 0;
  return static_cast<size_t>(n);
}

// Validates decode attention and fills its kernel arguments (a.M == 0 on return:
// nothing to launch).
static a8w8_status make_attn_args(const uint16_t* q_bf16, int64_t M, int n_q_heads,
                                  int n_kv_heads, int head_dim, const uint16_t* k_cache_bf16,
                                  const uint16_t* v_cache_bf16, int64_t num_blocks,
                                  int64_t block_size, const int32_t* block_table,
                                  int64_t blocks_per_seq, const int32_t* context_lens,
                                  float scale, uint16_t* out_bf16, void* workspace,
                                  size_t ws_bytes, AttnArgs& a) {
  if (num_blocks <= 0 || block_size <= 0 || blocks_per_seq <= 0 ||
      num_blocks > (int64_t(1) << 31) - 1 || block_size > (int64_t(1) << 31) - 1 ||
      blocks_per_seq > (int64_t(1) << 30) / block_size ||
      !attn_shapes_ok(M, n_q_heads, n_kv_heads, head_dim, blocks_per_seq * block_size))
    return A8W8_ERR_SHAPE;
  if (M == 0) {
    a = AttnArgs{};
    return A8W8_OK;
  }
  if (!q_bf16 || !k_cache_bf16 || !v_cache_bf16 || !block_table || !context_lens || !out_bf16)
    return A8W8_ERR_NULL;
  if (!aligned16(q_bf16) || !aligned16(out_bf16) || !aligned16(k_cache_bf16) ||
      !aligned16(v_cache_bf16) ||
      ((reinterpret_cast<uintptr_t>(block_table) | reinterpret_cast<uintptr_t>(context_lens)) & 3u))
    return A8W8_ERR_ALIGN;
  const int64_t max_ctx = blocks_per_seq * block_size;
  a = AttnArgs{};
  a.q = q_bf16;
  a.M = M;
  a.ld_q = int64_t(n_q_heads) * head_dim;
  a.n_q = n_q_heads;
  a.n_kv = n_kv_heads;
  a.group = n_q_heads / n_kv_heads;
  a.head_dim = head_dim;
  a.k_cache = k_cache_bf16;
  a.v_cache = v_cache_bf16;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.block_table = block_table;
  a.blocks_per_seq = blocks_per_seq;
  a.context_lens = context_lens;
  a.scale = scale;
  a.out = out_bf16;
  if (workspace == nullptr) {
    a.split_len = (max_ctx + 63) / 64 * 64;  // one split: no workspace needed
  } else {
    a.split_len = attn_split_len(M, n_kv_heads, max_ctx);
  }
  a.n_split = (max_ctx + a.split_len - 1) / a.split_len;
  if (attn_whole(M, n_kv_heads, max_ctx))
    a.waves = 8;  // eight waves on whole chunks
  else
    a.waves = (M * n_kv_heads * ((max_ctx + 63) / 64) < kAttnFourWaveChunks) ? 4 : 1;
  if (a.n_split > 1) {
    const size_t need =
        a8w8_decode_attention_workspace_bytes(M, n_q_heads, n_kv_heads, head_dim, max_ctx);
    if (need == 0) return A8W8_ERR_SHAPE;  // partials beyond the addressable range
    if (ws_bytes < need) return A8W8_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return A8W8_ERR_ALIGN;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = a.ws_o + M * n_q_heads * a.n_split * head_dim;
  }
  return A8W8_OK;
}

a8w8_status a8w8_decode_attention(const uint16_t* q_bf16, int64_t M, int n_q_heads,
                                  int n_kv_heads, int head_dim, const uint16_t* k_cache_bf16,
                                  const uint16_t* v_cache_bf16, int64_t num_blocks,
                                  int64_t block_size, const int32_t* block_table,
                                  int64_t blocks_per_seq, const int32_t* context_lens,
                                  float scale, uint16_t* out_bf16, void* workspace,
                                  size_t ws_bytes, void* stream) {
  AttnArgs a;
  if (a8w8_status e = make_attn_args(q_bf16, M, n_q_heads, n_kv_heads, head_dim, k_cache_bf16,
                                     v_cache_bf16, num_blocks, block_size, block_table,
                                     blocks_per_seq, context_lens, scale, out_bf16, workspace,
                                     ws_bytes, a))
    return e;
  if (a.M == 0) return A8W8_OK;
  A8W8_HIP(launch_decode_attention(a, static_cast<hipStream_t>(stream)));
  return A8W8_OK;
}

}  // extern "C"
