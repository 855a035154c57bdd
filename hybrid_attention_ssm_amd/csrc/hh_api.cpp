// C ABI of libhymba_hh: argument validation, workspace layout and the launch
// sequence of each entry point.  Every check runs on the host before the
// first launch, so a rejected call touches no buffer.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/hh.h"
#include "hh_internal.h"

namespace {

thread_local std::string g_err;

hh_status fail(hh_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
hh_status fail(hh_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

// ---- optional per-stage event timing ---------------------------------------
struct TimingRec {
  const char *stage;
  hipEvent_t start, stop;
};
struct Timing {
  bool on = false;
  std::vector<TimingRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
thread_local Timing g_timing;

// Test aid: with HH_FAULT_INJECT set to a stage's name, that stage reports a
// failed launch without launching anything (a host-side stand-in for a launch
// error: the error path runs, no kernel is enqueued, nothing faults).
thread_local const char *g_injected_stage = nullptr;
bool fault_injected(const char *stage) {
  const char *v = std::getenv("HH_FAULT_INJECT");
  return v && std::strcmp(v, stage) == 0;
}

// Brackets one stage's launches with events when timing is enabled; run()
// performs the launches unless a fault is injected for this stage.
struct Stage {
  hipStream_t st;
  const char *name;
  TimingRec rec{nullptr, nullptr, nullptr};
  template <class F>
  hipError_t run(F &&launch) {
    if (fault_injected(name)) {
      g_injected_stage = name;
      return hipErrorLaunchFailure;
    }
    return launch();
  }
  Stage(hipStream_t s, const char *nm) : st(s), name(nm) {
    if (!g_timing.on) return;
    rec.stage = name;
    rec.start = g_timing.get();
    rec.stop = g_timing.get();
    if (rec.start) (void)hipEventRecord(rec.start, st);
  }
  ~Stage() {
    if (!rec.stage || !rec.start || !rec.stop) return;
    (void)hipEventRecord(rec.stop, st);
    g_timing.recs.push_back(rec);
  }
};

hh_status hip_fail(hipError_t e, const char *where) {
  if (g_injected_stage) {
    const char *stage = g_injected_stage;
    g_injected_stage = nullptr;
    return fail(HH_ERR_HIP, "%s: launch failure injected at stage '%s' (HH_FAULT_INJECT)", where, stage);
  }
  return fail(HH_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void *p) { return p && ((uintptr_t)p & 15u) == 0; }

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Shape {
  int d, H, G, hd, D, N, k, m, Wa, KV, n_in, dtype;
  int S, dtw;   // Mamba2 SSM heads (0: Mamba) and the dt block's width (S or D)
  size_t es;
  float eps, rope_base;
};

hh_status check_dims(const hh_dims *dm, int kv_producer, Shape &s) {
  if (!dm) return fail(HH_ERR_INVALID_ARG, "dims is NULL");
  if (dm->dtype != HH_F32 && dm->dtype != HH_BF16)
    return fail(HH_ERR_INVALID_ARG, "dtype %d is neither HH_F32 nor HH_BF16", dm->dtype);
  if (dm->d_model <= 0 || dm->n_heads <= 0 || dm->n_kv_heads <= 0 || dm->head_dim <= 0 ||
      dm->d_inner <= 0 || dm->d_state <= 0 || dm->d_conv <= 0 || dm->n_meta < 0)
    return fail(HH_ERR_INVALID_ARG, "dimensions must be positive (n_meta >= 0)");
  if (dm->n_heads % dm->n_kv_heads)
    return fail(HH_ERR_INVALID_ARG, "n_heads %d is not a multiple of n_kv_heads %d",
                dm->n_heads, dm->n_kv_heads);
  if (dm->n_heads / dm->n_kv_heads > 8)
    return fail(HH_ERR_UNSUPPORTED, "more than 8 query heads per KV head");
  if (dm->dtype == HH_BF16 ? dm->head_dim != 64 : (dm->head_dim != 32 && dm->head_dim != 64))
    return fail(HH_ERR_UNSUPPORTED, "head_dim %d not supported for this dtype", dm->head_dim);
  if (dm->d_state != 16) return fail(HH_ERR_UNSUPPORTED, "d_state %d (only 16)", dm->d_state);
  if (dm->d_conv < 2 || dm->d_conv > 4)
    return fail(HH_ERR_UNSUPPORTED, "d_conv %d (2..4 supported)", dm->d_conv);
  if (dm->d_model % 8 || dm->d_inner % 8 || (dm->n_heads * dm->head_dim) % 8)
    return fail(HH_ERR_UNSUPPORTED, "d_model, d_inner and n_heads*head_dim must be multiples of 8");
  if (dm->dtype == HH_BF16 && (dm->d_model % 64 || (dm->n_heads * dm->head_dim + dm->d_inner) % 64))
    return fail(HH_ERR_UNSUPPORTED, "bf16 path needs d_model and n_heads*head_dim + d_inner "
                                    "to be multiples of 64");
  // the row kernels hold a row in at most 2048 vector chunks per workgroup
  // (the decode norm's split merge, the block's pre-norms): 16384 values in
  // bf16, 8192 in fp32
  {
    const long widest = std::max<long>(std::max<long>(dm->d_model, (long)dm->n_heads * dm->head_dim),
                                       dm->d_inner);
    const long limit = dm->dtype == HH_BF16 ? 16384 : 8192;
    if (widest > limit)
      return fail(HH_ERR_UNSUPPORTED, "d_model, n_heads*head_dim and d_inner must be at most %ld for this "
                  "dtype (widest is %ld)", limit, widest);
  }
  if (!(dm->rms_eps >= 0.0f) || dm->rms_eps > 1.0f)
    return fail(HH_ERR_INVALID_ARG, "rms_eps must be in [0, 1]");
  if (!(dm->rope_base == 0.0f || (dm->rope_base > 1.0f && dm->rope_base < 1e30f)))
    return fail(HH_ERR_INVALID_ARG, "rope_base must be 0 (no rotary embedding) or a finite base > 1");
  if (dm->ssm_heads < 0 || (dm->ssm_heads > 0 && (dm->d_inner % dm->ssm_heads || dm->ssm_heads % 4)))
    return fail(HH_ERR_INVALID_ARG, "ssm_heads %d must be 0 or divide d_inner %d and be a multiple of 4",
                dm->ssm_heads, dm->d_inner);
  s.d = dm->d_model; s.H = dm->n_heads; s.G = dm->n_kv_heads; s.hd = dm->head_dim;
  s.D = dm->d_inner; s.N = dm->d_state; s.k = dm->d_conv; s.m = dm->n_meta;
  s.S = dm->ssm_heads;
  s.dtw = s.S ? s.S : s.D;
  s.Wa = s.H * s.hd;
  s.KV = kv_producer ? s.G * s.hd : 0;
  s.n_in = s.Wa + 2 * s.KV + 2 * s.D + s.dtw + 2 * s.N;
  s.dtype = dm->dtype;
  s.es = dm->dtype == HH_BF16 ? 2 : 4;
  s.eps = dm->rms_eps;
  s.rope_base = dm->rope_base;
  return HH_OK;
}

// rotary embedding of the in-projection: pair i turns by pos * f0 * ratio^i
// revolutions (f0 = 1/(2 pi), ratio = base^(-2/hd), in double)
void set_rope(hh::InProjOut &e, const Shape &s, int len_bias) {
  e.rope_base = s.rope_base;
  e.rope_m = s.m;
  e.len_bias = len_bias;
  e.rope_f0 = 0.15915494309189533577;
  e.rope_ratio = s.rope_base != 0.0f ? std::pow((double)s.rope_base, -2.0 / s.hd) : 1.0;
}

hh_status check_weights(const hh_weights *w, const Shape &s) {
  if (!w) return fail(HH_ERR_INVALID_ARG, "weights is NULL");
  if (!w->w_in || !w->dt_bias || !w->A || !w->conv_w || !w->conv_b || !w->beta_attn ||
      !w->beta_ssm || !w->w_out)
    return fail(HH_ERR_INVALID_ARG, "a weight pointer is NULL");
  if (!aligned16(w->w_in) || !aligned16(w->w_out))
    return fail(HH_ERR_INVALID_ARG, "w_in and w_out must be 16-byte aligned");
  (void)s;
  return HH_OK;
}

// ---- workspace layouts ----------------------------------------------------
struct PrefillLayout {
  size_t off[HH_WS_COUNT];
  size_t total;
  int chunk;
};

PrefillLayout prefill_layout(const Shape &s, int B, int n) {
  PrefillLayout L;
  const size_t T = (size_t)B * n;
  size_t o = 0;
  auto take = [&](int id, size_t bytes) { L.off[id] = o; o = up256(o + bytes); };
  for (int i = 0; i < HH_WS_COUNT; ++i) L.off[i] = SIZE_MAX;
  take(HH_WS_Q, T * s.Wa * s.es);
  if (s.KV) {
    take(HH_WS_K, (size_t)B * s.G * n * s.hd * s.es);
    take(HH_WS_V, (size_t)B * s.G * n * s.hd * s.es);
  }
  // the SSM features in the channel-block-major layout (whole 64-column blocks)
  const size_t D64 = (s.D + 63) / 64 * 64, dt64 = (s.dtw + 63) / 64 * 64;
  take(HH_WS_XS, T * D64 * 4);
  take(HH_WS_Z, T * D64 * s.es);
  take(HH_WS_DELTA, T * dt64 * 4);
  take(HH_WS_BC, T * 2 * s.N * 4);
  take(HH_WS_O, T * s.Wa * s.es);
  take(HH_WS_Y, T * s.D * s.es);
  take(HH_WS_F, T * (s.Wa + s.D) * s.es);
  take(HH_WS_SCAN, hh::scan_carry_bytes(B, n, s.D, s.N, &L.chunk));
  take(HH_WS_SSQ, T * (s.G + (s.D + 63) / 64) * 4);
  const size_t gp = s.dtype == HH_BF16
                        ? std::max(hh::skinny_part_bytes((int)T, s.d, s.n_in),
                                   hh::skinny_part_bytes((int)T, s.Wa + s.D, s.d))
                        : 0;
  if (gp) take(HH_WS_GEMM, gp);
  L.total = o;
  return L;
}

struct DecodeLayout {
  size_t q, xs, z, dt, bc, o, y, f, part, gemm, total;
  int split, nsplit;
};

DecodeLayout decode_layout(const Shape &s, int B, int max_real) {
  DecodeLayout L;
  size_t o = 0;
  auto take = [&](size_t &dst, size_t bytes) { dst = o; o = up256(o + bytes); };
  take(L.q, (size_t)B * s.Wa * s.es);
  take(L.xs, (size_t)B * s.D * 4);
  take(L.z, (size_t)B * s.D * s.es);
  take(L.dt, (size_t)B * s.dtw * 4);
  take(L.bc, (size_t)B * 2 * s.N * 4);
  take(L.o, (size_t)B * s.Wa * s.es);
  take(L.y, (size_t)B * s.D * s.es);
  take(L.f, (size_t)B * (s.Wa + s.D) * s.es);
  take(L.part, hh::decode_attn_part_bytes(B, s.H, s.G, s.hd, s.m, max_real, &L.split, &L.nsplit));
  L.gemm = SIZE_MAX;
  const size_t gp = s.dtype == HH_BF16 ? std::max(hh::skinny_part_bytes(B, s.d, s.n_in),
                                                  hh::skinny_part_bytes(B, s.Wa + s.D, s.d))
                                       : 0;
  if (gp) take(L.gemm, gp);
  L.total = o;
  return L;
}

char *at(void *ws, size_t off) { return static_cast<char *>(ws) + off; }

float *part_ptr(void *ws, size_t off) {
  return off == SIZE_MAX ? nullptr : reinterpret_cast<float *>(at(ws, off));
}

template <class T>
hh_status run_inproj(const Shape &s, const hh_weights *w, const void *x, int M,
                     const hh::InProjOut &e, float *part, hipStream_t st) {
  Stage sg(st, e.mode == hh::EPI_DECODE ? "decode_inproj"
              : e.mode == hh::EPI_META ? "meta_inproj" : "inproj");
  hipError_t err = sg.run([&] {
    return hh::launch_inproj<T>(static_cast<const T *>(x), M, s.d, static_cast<const T *>(w->w_in), s.n_in, e,
                                part, st);
  });
  return err == hipSuccess ? HH_OK : hip_fail(err, "input projection");
}

// ---- the SSM branch beside the attention branch ---------------------------
// A second stream per (host thread, device) with the default priority and
// three ordering events, created on the first prefill that uses it and
// destroyed when the thread ends.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t rows_a = nullptr, rows_b = nullptr, done = nullptr;
  ~SideStream() {
    if (rows_a) (void)hipEventDestroy(rows_a);
    if (rows_b) (void)hipEventDestroy(rows_b);
    if (done) (void)hipEventDestroy(done);
    if (s) (void)hipStreamDestroy(s);
  }
};
constexpr int kMaxSideDevices = 64;
thread_local SideStream g_side[kMaxSideDevices];

hh_status side_stream(SideStream **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxSideDevices)
    return fail(HH_ERR_UNSUPPORTED, "device %d: side streams are kept for devices 0..%d", dev,
                kMaxSideDevices - 1);
  SideStream &ss = g_side[dev];
  if (!ss.s) {
    SideStream fresh;
    if ((e = hipStreamCreateWithFlags(&fresh.s, hipStreamNonBlocking)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&fresh.rows_a, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&fresh.rows_b, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&fresh.done, hipEventDisableTiming)) != hipSuccess)
      return hip_fail(e, "side stream set-up");
    std::swap(ss.s, fresh.s);
    std::swap(ss.rows_a, fresh.rows_a);
    std::swap(ss.rows_b, fresh.rows_b);
    std::swap(ss.done, fresh.done);
  }
  *out = &ss;
  return HH_OK;
}

// The two branches run side by side only when HH_CONCURRENT_BRANCHES=1.  It
// is off by default: measured on the 8k prefill, the scan's waves beside the
// second half of the input projection slow that GEMM by about a quarter (the
// two compete for LDS bandwidth and issue slots; raising the GEMM waves'
// priority changed nothing), and beside the attention they slow it as much
// as they gain, so the step takes 0.88 ms against 0.85 ms in one stream.
bool concurrent_branches(const Shape &, long) {
  const char *v = std::getenv("HH_CONCURRENT_BRANCHES");
  return v && v[0] == '1';
}

// The attention and scan pass 3 in one launch whose workgroups take either
// role (bf16, HH_ONE_LAUNCH_BRANCHES=1): the same arithmetic as the two
// kernels one after the other, so the same results bit for bit.  Off by
// default: on the 8k prefill the shared grid takes 250 us against 117 + 125 us
// for the two kernels.  Each kernel alone already fills a CU's registers and
// LDS, both hide latency with their wave count, and the scan's VALU work plus
// the softmax's exceed the VALU issue rate, so sharing CUs only splits them.
bool one_launch_branches(const Shape &s) {
  const char *v = std::getenv("HH_ONE_LAUNCH_BRANCHES");
  return v && v[0] == '1' && s.dtype == HH_BF16;
}

// The fusion of Eq. (3) inside the output projection (bf16, many rows): the
// branches store beta-scaled outputs and per-row sums of squares, and the
// GEMM applies the row scales to its accumulators, so no normalised copy of
// the features is written or read.  HH_FUSED_NORM=0 selects the separate
// norm kernel instead (same result up to where the bf16 roundings fall).
bool fused_norm(const Shape &s, int rows) {
  const char *v = std::getenv("HH_FUSED_NORM");
  if (v && v[0] == '0') return false;
  return s.dtype == HH_BF16 && hh::outproj_fused_ok(rows, s.Wa, s.D);
}

// Prefill.  With the branches side by side (concurrent_branches), the input
// projection runs in two row ranges on the caller's stream; the SSM branch's
// chunk summaries (scan pass 1) of the first range start on the side stream as
// soon as that range is projected and run beside the second range's
// projection, whose matrix-core work leaves the vector ALUs mostly idle; the
// rest of the scan runs beside the attention branch; the caller's stream
// waits for it before the fusion.  Every kernel computes what it computes in
// the single-stream order, so the results are the same bit for bit.
template <class T>
hh_status prefill_t(const Shape &s, const hh_weights *w, const void *x, int B, int n,
                    const hh_meta *meta, int window, int is_global, void *out, hh_kv *kv,
                    hh_ssm_state *state, void *ws, const PrefillLayout &L, hipStream_t st,
                    const void *resid = nullptr) {
  const int rows = B * n;
  const bool prod = w->kv_producer != 0;
  void *kfull = prod ? ((kv && kv->full_k) ? kv->full_k : at(ws, L.off[HH_WS_K])) : kv->full_k;
  void *vfull = prod ? ((kv && kv->full_v) ? kv->full_v : at(ws, L.off[HH_WS_V])) : kv->full_v;

  hh::InProjOut e{};
  e.mode = hh::EPI_PREFILL;
  e.Wa = s.Wa; e.KV = s.KV; e.D = s.D; e.Ddt = s.dtw; e.N = s.N; e.hd = s.hd; e.n_rows_per_seq = n;
  e.q = at(ws, L.off[HH_WS_Q]);
  e.k_full = kfull; e.v_full = vfull;
  if (prod && kv && kv->cache_k) {
    e.cache_k = kv->cache_k; e.cache_v = kv->cache_v; e.cap = kv->cap; e.is_ring = kv->is_ring;
  }
  e.ssm_rows = rows;
  e.xs = reinterpret_cast<float *>(at(ws, L.off[HH_WS_XS])); e.z = at(ws, L.off[HH_WS_Z]);
  e.dt = reinterpret_cast<float *>(at(ws, L.off[HH_WS_DELTA]));
  e.bc = reinterpret_cast<float *>(at(ws, L.off[HH_WS_BC]));
  e.dt_bias = w->dt_bias;
  set_rope(e, s, 0);

  hh::ScanArgs sa{};
  sa.xs = e.xs; sa.z = e.z; sa.dt = e.dt; sa.bc = e.bc;
  sa.A = w->A; sa.conv_w = w->conv_w; sa.conv_b = w->conv_b;
  sa.h0 = meta->h0; sa.tail0 = meta->conv_tail;
  sa.y = at(ws, L.off[HH_WS_Y]);
  sa.h_out = state ? state->h : nullptr;
  sa.tail_out = state ? state->conv : nullptr;
  sa.carry = reinterpret_cast<float *>(at(ws, L.off[HH_WS_SCAN]));
  sa.B = B; sa.n = n; sa.D = s.D; sa.N = s.N; sa.k = s.k; sa.S = s.S; sa.chunk = L.chunk;
  const bool fused = fused_norm(s, rows);
  float *ssq_o = reinterpret_cast<float *>(at(ws, L.off[HH_WS_SSQ]));
  float *ssq_y = ssq_o + (size_t)rows * s.G;
  if (fused) { sa.beta = w->beta_ssm; sa.ssq = ssq_y; }

  // the first row range: whole sequences when there are several, else the
  // rows of the first half of the chunks that have summaries
  SideStream *side = nullptr;
  int rows_a = 0, ck_a = 0, b_a = 0;
  const int nchunks = hh::scan_chunks(sa);
  if (concurrent_branches(s, rows)) {
    if (B >= 2) { b_a = B / 2; rows_a = b_a * n; }
    else { ck_a = (nchunks - 1) / 2; rows_a = ck_a * L.chunk; }
    if (rows_a > 0) {
      hh_status r = side_stream(&side);
      if (r != HH_OK) return r;
    }
  }
  hipError_t err;
  float *gemm_part = part_ptr(ws, L.off[HH_WS_GEMM]);
  if (!side) {
    hh_status r = run_inproj<T>(s, w, x, rows, e, gemm_part, st);
    if (r != HH_OK) return r;
  } else {
    // the two row ranges (one GEMM each) on the caller's stream, an event after each
    {
      Stage sg(st, "inproj");
      err = sg.run([&] {
        hipError_t q = hh::launch_inproj<T>(static_cast<const T *>(x), rows_a, s.d,
                                            static_cast<const T *>(w->w_in), s.n_in, e, gemm_part, st);
        if (q == hipSuccess) q = hipEventRecord(side->rows_a, st);
        hh::InProjOut eb = e;
        eb.row0 = rows_a;
        if (q == hipSuccess)
          q = hh::launch_inproj<T>(static_cast<const T *>(x) + (size_t)rows_a * s.d, rows - rows_a, s.d,
                                   static_cast<const T *>(w->w_in), s.n_in, eb, gemm_part, st);
        if (q == hipSuccess) q = hipEventRecord(side->rows_b, st);
        return q;
      });
    }
    if (err != hipSuccess) return hip_fail(err, "input projection");
    // the SSM branch on the side stream
    {
      Stage sg(side->s, "scan");
      err = sg.run([&] {
        hipError_t q = hipStreamWaitEvent(side->s, side->rows_a, 0);
        if (q == hipSuccess)
          q = B >= 2 ? hh::launch_scan_summaries<T>(sa, 0, nchunks, 0, b_a, side->s)
                     : hh::launch_scan_summaries<T>(sa, 0, ck_a, 0, 1, side->s);
        if (q == hipSuccess) q = hipStreamWaitEvent(side->s, side->rows_b, 0);
        if (q == hipSuccess)
          q = B >= 2 ? hh::launch_scan_summaries<T>(sa, 0, nchunks, b_a, B, side->s)
                     : hh::launch_scan_summaries<T>(sa, ck_a, nchunks, 0, 1, side->s);
        if (q == hipSuccess) q = hh::launch_scan_finish<T>(sa, side->s);
        if (q == hipSuccess) q = hipEventRecord(side->done, side->s);
        return q;
      });
    }
    if (err != hipSuccess) return hip_fail(err, "selective scan");
  }

  hh::AttnArgs aa{};
  aa.q = e.q; aa.k = kfull; aa.v = vfull; aa.mk = meta->k; aa.mv = meta->v;
  aa.o = at(ws, L.off[HH_WS_O]);
  aa.B = B; aa.n = n; aa.m = s.m; aa.H = s.H; aa.G = s.G; aa.hd = s.hd;
  aa.window = window; aa.is_global = is_global;
  const bool set_len = prod && kv && kv->len;   // the cache now holds the prompt's n positions
  if (fused) {
    aa.beta = w->beta_attn; aa.ssq = ssq_o;
    if (set_len) { aa.set_len = kv->len; aa.set_len_n = B; aa.set_len_value = n; }
  }
  const bool one_launch = !side && one_launch_branches(s);   // read once per call
  if (one_launch) {
    // scan passes 1 and 2, then the attention beside scan pass 3
    {
      Stage sg(st, "scan_carries");
      err = sg.run([&] {
        hipError_t q = hh::launch_scan_summaries<T>(sa, 0, nchunks, 0, B, st);
        return q == hipSuccess ? hh::launch_scan_carries<T>(sa, st) : q;
      });
    }
    if (err != hipSuccess) return hip_fail(err, "selective scan");
    {
      Stage sg(st, "attention_scan");
      err = sg.run([&] { return hh::launch_attn_scan3<T>(aa, sa, st); });
    }
    if (err != hipSuccess) return hip_fail(err, "attention and selective scan");
  } else {
    {
      Stage sg(st, "attention");
      err = sg.run([&] { return hh::launch_attention<T>(aa, st); });
    }
    if (err != hipSuccess) return hip_fail(err, "attention");
  }

  if (one_launch) {
    // done above
  } else if (!side) {
    {
      Stage sg(st, "scan");
      err = sg.run([&] { return hh::launch_scan<T>(sa, st); });
    }
    if (err != hipSuccess) return hip_fail(err, "selective scan");
  } else if ((err = hipStreamWaitEvent(st, side->done, 0)) != hipSuccess) {
    return hip_fail(err, "joining the SSM branch");
  }

  if (fused) {
    const hh::NormScale ns{sa.y, ssq_o, ssq_y, s.Wa, s.D, s.G, (s.D + 63) / 64, s.eps};
    Stage sg(st, "outproj");
    err = sg.run([&] {
      return hh::launch_outproj_fused<T>(static_cast<const T *>(aa.o), ns, rows,
                                         static_cast<const T *>(w->w_out), s.d, static_cast<T *>(out),
                                         static_cast<const T *>(resid), st);
    });
    if (err != hipSuccess) return hip_fail(err, "output projection");
    return HH_OK;
  }

  hh::NormArgs na{};
  na.o = aa.o; na.y = sa.y; na.beta_attn = w->beta_attn; na.beta_ssm = w->beta_ssm;
  na.f = at(ws, L.off[HH_WS_F]);
  na.rows = rows; na.Wa = s.Wa; na.D = s.D; na.eps = s.eps;
  if (set_len) { na.set_len = kv->len; na.set_len_n = B; na.set_len_value = n; }
  {
    Stage sg(st, "norm");
    err = sg.run([&] { return hh::launch_norm_fuse<T>(na, st); });
  }
  if (err != hipSuccess) return hip_fail(err, "norm/average");

  {
    Stage sg(st, "outproj");
    err = sg.run([&] {
      return hh::launch_outproj<T>(static_cast<const T *>(na.f), rows, s.Wa + s.D,
                                   static_cast<const T *>(w->w_out), s.d, static_cast<T *>(out),
                                   static_cast<const T *>(resid), gemm_part, st);
    });
  }
  if (err != hipSuccess) return hip_fail(err, "output projection");

  return HH_OK;
}

template <class T>
hh_status meta_prefix_t(const Shape &s, const hh_weights *w, const void *R, void *mk, void *mv,
                        float *h0, float *tail, void *ws, const PrefillLayout &L, hipStream_t st) {
  hh::InProjOut e{};
  e.mode = hh::EPI_META;
  e.Wa = s.Wa; e.KV = s.KV; e.D = s.D; e.Ddt = s.dtw; e.N = s.N; e.hd = s.hd; e.n_rows_per_seq = s.m;
  e.q = at(ws, L.off[HH_WS_Q]);
  e.k_full = mk; e.v_full = mv;
  e.ssm_rows = s.m;
  e.xs = reinterpret_cast<float *>(at(ws, L.off[HH_WS_XS])); e.z = at(ws, L.off[HH_WS_Z]);
  e.dt = reinterpret_cast<float *>(at(ws, L.off[HH_WS_DELTA]));
  e.bc = reinterpret_cast<float *>(at(ws, L.off[HH_WS_BC]));
  e.dt_bias = w->dt_bias;
  set_rope(e, s, 0);
  hh_status r = run_inproj<T>(s, w, R, s.m, e, part_ptr(ws, L.off[HH_WS_GEMM]), st);
  if (r != HH_OK) return r;
  hh::ScanArgs sa{};
  sa.xs = e.xs; sa.z = nullptr; sa.dt = e.dt; sa.bc = e.bc;
  sa.A = w->A; sa.conv_w = w->conv_w; sa.conv_b = w->conv_b;
  sa.h0 = nullptr; sa.tail0 = nullptr; sa.y = nullptr;
  sa.h_out = h0; sa.tail_out = tail;
  sa.carry = reinterpret_cast<float *>(at(ws, L.off[HH_WS_SCAN]));
  sa.B = 1; sa.n = s.m; sa.D = s.D; sa.N = s.N; sa.k = s.k; sa.S = s.S; sa.chunk = L.chunk;
  Stage sg(st, "meta_scan");
  hipError_t err = sg.run([&] { return hh::launch_scan<T>(sa, st); });
  return err == hipSuccess ? HH_OK : hip_fail(err, "meta scan");
}

template <class T>
hh_status decode_t(const Shape &s, const hh_weights *w, const void *x, int B, const hh_meta *meta,
                   int window, int is_global, hh_kv *kv, hh_ssm_state *state, void *out, void *ws,
                   const DecodeLayout &L, hipStream_t st, const void *resid = nullptr) {
  const bool prod = w->kv_producer != 0;
  hh::InProjOut e{};
  e.mode = hh::EPI_DECODE;
  e.Wa = s.Wa; e.KV = s.KV; e.D = s.D; e.Ddt = s.dtw; e.N = s.N; e.hd = s.hd; e.n_rows_per_seq = 1;
  e.q = at(ws, L.q);
  e.cache_k = kv->cache_k; e.cache_v = kv->cache_v; e.cap = kv->cap; e.is_ring = kv->is_ring;
  e.len = kv->len;
  e.xs = reinterpret_cast<float *>(at(ws, L.xs)); e.z = at(ws, L.z);
  e.dt = reinterpret_cast<float *>(at(ws, L.dt));
  e.bc = reinterpret_cast<float *>(at(ws, L.bc));
  e.dt_bias = w->dt_bias;
  set_rope(e, s, prod ? 0 : -1);
  hh_status r = run_inproj<T>(s, w, x, B, e, part_ptr(ws, L.gemm), st);
  if (r != HH_OK) return r;

  hh::DecodeAttnArgs da{};
  da.q = e.q; da.cache_k = kv->cache_k; da.cache_v = kv->cache_v;
  da.mk = meta->k; da.mv = meta->v; da.len = kv->len; da.producer = prod ? 1 : 0;
  da.o = at(ws, L.o);
  da.part = reinterpret_cast<float *>(at(ws, L.part));
  da.B = B; da.H = s.H; da.G = s.G; da.hd = s.hd; da.m = s.m; da.cap = kv->cap;
  da.is_ring = kv->is_ring; da.window = window; da.is_global = is_global;
  da.split = L.split;
  da.nsplit = L.nsplit;
  hh::DecodeSsmArgs sa{};
  sa.xs = e.xs; sa.z = e.z; sa.dt = e.dt; sa.bc = e.bc;
  sa.A = w->A; sa.conv_w = w->conv_w; sa.conv_b = w->conv_b;
  sa.h = state->h; sa.conv = state->conv; sa.y = at(ws, L.y);
  sa.B = B; sa.D = s.D; sa.N = s.N; sa.k = s.k; sa.S = s.S;
  hipError_t err;
  bool o_ready = false;
  {
    Stage sg(st, is_global ? "decode_attention_global" : "decode_attention_swa");
    err = sg.run([&] { return hh::launch_decode_attention<T>(da, st, &o_ready); });
  }
  if (err != hipSuccess) return hip_fail(err, "decode attention");
  {
    Stage sg(st, "decode_ssm");
    err = sg.run([&] { return hh::launch_decode_ssm<T>(sa, st); });
  }
  if (err != hipSuccess) return hip_fail(err, "decode SSM step");

  hh::NormArgs na{};
  na.o = da.o; na.y = sa.y; na.beta_attn = w->beta_attn; na.beta_ssm = w->beta_ssm;
  na.f = at(ws, L.f);
  na.rows = B; na.Wa = s.Wa; na.D = s.D; na.eps = s.eps;
  if (prod) {   // the new token joins the producer's cache after this step's attention
    na.len_bump = kv->len; na.bump_n = B; na.bump_cap = kv->cap; na.bump_ring = kv->is_ring;
  }
  if (!o_ready) {   // merge the attention's split partials here
    na.part = da.part; na.H = s.H; na.hd = s.hd; na.nsplit = da.nsplit;
  }
  {
    Stage sg(st, "decode_norm");
    err = sg.run([&] { return hh::launch_norm_fuse<T>(na, st); });
  }
  if (err != hipSuccess) return hip_fail(err, "decode norm/average");

  {
    Stage sg(st, "decode_outproj");
    err = sg.run([&] {
      return hh::launch_outproj<T>(static_cast<const T *>(na.f), B, s.Wa + s.D,
                                   static_cast<const T *>(w->w_out), s.d, static_cast<T *>(out),
                                   static_cast<const T *>(resid), part_ptr(ws, L.gemm), st);
    });
  }
  if (err != hipSuccess) return hip_fail(err, "decode output projection");
  return HH_OK;
}

int max_real_keys(const hh_kv *kv, int window, int is_global) {
  if (is_global || !kv->is_ring) return kv->cap;
  return std::min(window, kv->cap);
}


// ---- argument checks shared by the layer and block entry points -----------
hh_status check_prefill_call(const hh_dims *dims, const hh_weights *w, const void *x, int batch,
                             int seqlen, const hh_meta *meta, int window, int is_global,
                             const void *out, const hh_kv *kv, Shape &s) {
  hh_status r = check_dims(dims, w ? w->kv_producer : 1, s);
  if (r != HH_OK) return r;
  if ((r = check_weights(w, s)) != HH_OK) return r;
  if (batch <= 0 || seqlen <= 0) return fail(HH_ERR_INVALID_ARG, "batch and seqlen must be positive");
  if ((long long)batch * seqlen > (1LL << 30))
    return fail(HH_ERR_UNSUPPORTED, "batch*seqlen above 2^30 tokens");
  if (!is_global && window < 1) return fail(HH_ERR_INVALID_ARG, "window must be >= 1");
  if (!aligned16(x) || !aligned16(out)) return fail(HH_ERR_INVALID_ARG, "x/out NULL or not 16-byte aligned");
  if (!meta) return fail(HH_ERR_INVALID_ARG, "meta is NULL");
  if (s.m > 0 && (!aligned16(meta->k) || !aligned16(meta->v)))
    return fail(HH_ERR_INVALID_ARG, "meta k/v NULL or not 16-byte aligned");
  if (!w->kv_producer) {
    if (!kv || !aligned16(kv->full_k) || !aligned16(kv->full_v))
      return fail(HH_ERR_INVALID_ARG, "a consumer layer needs its producer's full_k/full_v");
  }
  if (w->kv_producer && kv) {
    if ((kv->full_k && !aligned16(kv->full_k)) || (kv->full_v && !aligned16(kv->full_v)) ||
        (!kv->full_k) != (!kv->full_v))
      return fail(HH_ERR_INVALID_ARG, "full_k/full_v must both be NULL or both 16-byte aligned");
    if ((!kv->cache_k) != (!kv->cache_v))
      return fail(HH_ERR_INVALID_ARG, "cache_k/cache_v must both be set or both NULL");
    if (kv->cache_k) {
      if (kv->cap < 1) return fail(HH_ERR_INVALID_ARG, "cache cap must be >= 1");
      if (kv->is_ring && is_global) return fail(HH_ERR_INVALID_ARG, "a global layer needs a linear cache");
      if (kv->is_ring && window > kv->cap)
        return fail(HH_ERR_INVALID_ARG, "ring cache cap %d below window %d", kv->cap, window);
      // a linear cache must hold every prompt position: the prompt's length
      // becomes len, and decode appends at slot len
      if (!kv->is_ring && kv->cap < seqlen)
        return fail(HH_ERR_INVALID_ARG, "linear cache cap %d below seqlen %d", kv->cap, seqlen);
    }
  }
  return HH_OK;
}

hh_status check_decode_call(const hh_dims *dims, const hh_weights *w, const void *x_t, int batch,
                            const hh_meta *meta, int window, int is_global, const hh_kv *kv,
                            const hh_ssm_state *state, const void *out, Shape &s) {
  hh_status r = check_dims(dims, w ? w->kv_producer : 1, s);
  if (r != HH_OK) return r;
  if ((r = check_weights(w, s)) != HH_OK) return r;
  if (batch <= 0) return fail(HH_ERR_INVALID_ARG, "batch must be positive");
  if (!is_global && window < 1) return fail(HH_ERR_INVALID_ARG, "window must be >= 1");
  if (!aligned16(x_t) || !aligned16(out)) return fail(HH_ERR_INVALID_ARG, "x_t/out NULL or not 16-byte aligned");
  if (!meta) return fail(HH_ERR_INVALID_ARG, "meta is NULL");
  if (s.m > 0 && (!aligned16(meta->k) || !aligned16(meta->v)))
    return fail(HH_ERR_INVALID_ARG, "meta k/v NULL or not 16-byte aligned");
  if (!kv || !aligned16(kv->cache_k) || !aligned16(kv->cache_v) || !kv->len)
    return fail(HH_ERR_INVALID_ARG, "decode needs cache_k, cache_v and len");
  if (kv->cap < 1) return fail(HH_ERR_INVALID_ARG, "cache cap must be >= 1");
  if (kv->is_ring && is_global) return fail(HH_ERR_INVALID_ARG, "a global layer needs a linear cache");
  if (kv->is_ring && window > kv->cap)
    return fail(HH_ERR_INVALID_ARG, "ring cache cap %d below window %d", kv->cap, window);
  if (!state || !aligned16(state->h) || !state->conv)
    return fail(HH_ERR_INVALID_ARG, "decode needs the SSM state h and conv");
  return HH_OK;
}


// ---- the block around the layer -------------------------------------------
struct BlockLayout {
  size_t n1, x1, n2, h, part, total;
};

// The block's buffers follow the layer's workspace (base bytes).
BlockLayout block_layout(const Shape &s, size_t base, size_t T, int d_ff) {
  BlockLayout L;
  size_t o = up256(base);
  auto take = [&](size_t &dst, size_t bytes) { dst = o; o = up256(o + bytes); };
  take(L.n1, T * s.d * s.es);
  take(L.x1, T * s.d * s.es);
  take(L.n2, T * s.d * s.es);
  take(L.h, T * d_ff * s.es);
  const size_t gp = s.dtype == HH_BF16 ? std::max(hh::skinny_part_bytes((int)T, s.d, 2 * d_ff),
                                                  hh::skinny_part_bytes((int)T, d_ff, s.d))
                                       : 0;
  L.part = SIZE_MAX;
  if (gp) take(L.part, gp);
  L.total = o;
  return L;
}

hh_status check_block_weights(const hh_block_weights *w) {
  if (!w) return fail(HH_ERR_INVALID_ARG, "block weights are NULL");
  if (!w->norm1 || !w->norm2) return fail(HH_ERR_INVALID_ARG, "norm1/norm2 NULL");
  if (!aligned16(w->w_gate_up) || !aligned16(w->w_down))
    return fail(HH_ERR_INVALID_ARG, "w_gate_up/w_down NULL or not 16-byte aligned");
  if (w->d_ff <= 0 || w->d_ff % 4)
    return fail(HH_ERR_UNSUPPORTED, "d_ff %d is not a positive multiple of 4", w->d_ff);
  return HH_OK;
}

// the bf16 GEMMs walk K in 64-wide k-tiles: the down projection's K is d_ff
hh_status check_block_shape(const hh_block_weights *w, const Shape &s) {
  if (s.dtype == HH_BF16 && w->d_ff % 64)
    return fail(HH_ERR_UNSUPPORTED, "bf16 path needs d_ff (%d) to be a multiple of 64", w->d_ff);
  return HH_OK;
}

// out = x1 + MLP(g2 * rms(x1)), x1 already in the block workspace
template <class T>
hh_status block_mlp_t(const Shape &s, const hh_block_weights *w, int rows, void *ws,
                      const BlockLayout &BL, void *out, hipStream_t st) {
  const T *x1 = reinterpret_cast<const T *>(at(ws, BL.x1));
  T *n2 = reinterpret_cast<T *>(at(ws, BL.n2));
  T *h = reinterpret_cast<T *>(at(ws, BL.h));
  float *part = part_ptr(ws, BL.part);
  hipError_t err;
  {
    Stage sg(st, "block_norm2");
    err = sg.run([&] { return hh::launch_rmsnorm<T>(x1, w->norm2, n2, rows, s.d, s.eps, st); });
  }
  if (err != hipSuccess) return hip_fail(err, "block pre-norm 2");
  {
    Stage sg(st, "mlp_gate_up");
    err = sg.run([&] {
      return hh::launch_mlp_gate_up<T>(n2, rows, s.d, static_cast<const T *>(w->w_gate_up), 2 * w->d_ff, h,
                                       part, st);
    });
  }
  if (err != hipSuccess) return hip_fail(err, "MLP gate/up projection");
  {
    Stage sg(st, "mlp_down");
    err = sg.run([&] {
      return hh::launch_outproj<T>(h, rows, w->d_ff, static_cast<const T *>(w->w_down), s.d,
                                   static_cast<T *>(out), x1, part, st);
    });
  }
  return err == hipSuccess ? HH_OK : hip_fail(err, "MLP down projection");
}

template <class T>
hh_status block_norm1_t(const Shape &s, const hh_block_weights *w, const void *x, int rows, void *dst,
                        hipStream_t st) {
  Stage sg(st, "block_norm1");
  hipError_t err = sg.run([&] {
    return hh::launch_rmsnorm<T>(static_cast<const T *>(x), w->norm1, static_cast<T *>(dst), rows, s.d, s.eps,
                                 st);
  });
  return err == hipSuccess ? HH_OK : hip_fail(err, "block pre-norm 1");
}

template <class T>
hh_status block_prefill_t(const Shape &s, const hh_block_weights *w, const void *x, int B, int n,
                          const hh_meta *meta, int window, int is_global, void *out, hh_kv *kv,
                          hh_ssm_state *state, void *ws, const PrefillLayout &L,
                          const BlockLayout &BL, hipStream_t st) {
  const int rows = B * n;
  hh_status r = block_norm1_t<T>(s, w, x, rows, at(ws, BL.n1), st);
  if (r != HH_OK) return r;
  r = prefill_t<T>(s, &w->mixer, at(ws, BL.n1), B, n, meta, window, is_global, at(ws, BL.x1), kv,
                   state, ws, L, st, x);
  if (r != HH_OK) return r;
  return block_mlp_t<T>(s, w, rows, ws, BL, out, st);
}

template <class T>
hh_status block_decode_t(const Shape &s, const hh_block_weights *w, const void *x, int B,
                         const hh_meta *meta, int window, int is_global, hh_kv *kv,
                         hh_ssm_state *state, void *out, void *ws, const DecodeLayout &L,
                         const BlockLayout &BL, hipStream_t st) {
  hh_status r = block_norm1_t<T>(s, w, x, B, at(ws, BL.n1), st);
  if (r != HH_OK) return r;
  r = decode_t<T>(s, &w->mixer, at(ws, BL.n1), B, meta, window, is_global, kv, state,
                  at(ws, BL.x1), ws, L, st, x);
  if (r != HH_OK) return r;
  return block_mlp_t<T>(s, w, B, ws, BL, out, st);
}

// ---- scratch of the entry point that allocates nothing ---------------------
// hh_decode_step_noalloc's workspace: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  In host code the
// array's name is not a device address; its address on the current device
// comes from hipGetSymbolAddress (once per device, kept in g_scratch) and is
// the only way the host refers to it.  No kernel of the decode step reads a
// scratch byte it has not written in the same call, so nothing is cleared.
constexpr size_t kStaticScratchBytes = HH_STATIC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxScratchDevices] = {};

hh_status static_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(HH_ERR_UNSUPPORTED, "device %d: the static scratch is tracked for devices 0..%d", dev,
                kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HH_OK;
}

}  // namespace

extern "C" {

const char *hh_version(void) { return "libhymba_hh 0.1.0 gfx950"; }

const char *hh_last_error(void) { return g_err.c_str(); }

hh_status hh_timing_enable(int32_t on) {
  g_timing.on = on != 0;
  return HH_OK;
}

int32_t hh_timing_read(hh_stage_time *out, int32_t max_stages) {
  std::vector<hh_stage_time> agg;
  int32_t rc = 0;
  for (TimingRec &r : g_timing.recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      rc = -1;
    size_t i = 0;
    while (i < agg.size() && std::strcmp(agg[i].name, r.stage) != 0) ++i;
    if (i == agg.size()) {
      hh_stage_time t{};
      std::snprintf(t.name, sizeof t.name, "%s", r.stage);
      agg.push_back(t);
    }
    agg[i].launches += 1;
    agg[i].total_ms += ms;
    g_timing.pool.push_back(r.start);
    g_timing.pool.push_back(r.stop);
  }
  g_timing.recs.clear();
  if (rc < 0) return rc;
  const int32_t n = std::min<int32_t>((int32_t)agg.size(), max_stages);
  for (int32_t i = 0; i < n && out; ++i) out[i] = agg[i];
  return n;
}

size_t hh_prefill_workspace_layout(const hh_dims *dims, int32_t batch, int32_t seqlen,
                                   int32_t kv_producer, size_t *offs) {
  Shape s;
  if (check_dims(dims, kv_producer, s) != HH_OK || batch <= 0 || seqlen <= 0) return 0;
  PrefillLayout L = prefill_layout(s, batch, seqlen);
  if (offs) std::memcpy(offs, L.off, sizeof L.off);
  return L.total;
}

size_t hh_prefill_workspace_size(const hh_dims *dims, int32_t batch, int32_t seqlen,
                                 int32_t kv_producer) {
  return hh_prefill_workspace_layout(dims, batch, seqlen, kv_producer, nullptr);
}

size_t hh_meta_prefix_workspace_size(const hh_dims *dims, int32_t kv_producer) {
  if (!dims || dims->n_meta <= 0) return 0;
  return hh_prefill_workspace_layout(dims, 1, dims->n_meta, kv_producer, nullptr);
}

size_t hh_decode_workspace_size(const hh_dims *dims, int32_t batch, int32_t cap,
                                int32_t kv_producer) {
  Shape s;
  if (check_dims(dims, kv_producer, s) != HH_OK || batch <= 0 || cap <= 0) return 0;
  return decode_layout(s, batch, cap).total;
}

hh_status hh_meta_prefix(const hh_dims *dims, const hh_weights *w, const void *meta_tokens,
                         void *meta_k, void *meta_v, float *h0, float *conv_tail, void *ws,
                         size_t ws_bytes, void *stream) {
  Shape s;
  hh_status r = check_dims(dims, w ? w->kv_producer : 1, s);
  if (r != HH_OK) return r;
  if ((r = check_weights(w, s)) != HH_OK) return r;
  if (s.m <= 0) return fail(HH_ERR_INVALID_ARG, "n_meta must be positive for hh_meta_prefix");
  if (!aligned16(meta_tokens)) return fail(HH_ERR_INVALID_ARG, "meta_tokens NULL or not 16-byte aligned");
  if (s.KV && (!meta_k || !meta_v)) return fail(HH_ERR_INVALID_ARG, "meta_k/meta_v NULL for a producer layer");
  if (!h0 || !conv_tail) return fail(HH_ERR_INVALID_ARG, "h0/conv_tail NULL");
  PrefillLayout L = prefill_layout(s, 1, s.m);
  if (!ws || ws_bytes < L.total)
    return fail(HH_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, L.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return s.dtype == HH_BF16 ? meta_prefix_t<hh::bf16>(s, w, meta_tokens, meta_k, meta_v, h0, conv_tail, ws, L, st)
                            : meta_prefix_t<float>(s, w, meta_tokens, meta_k, meta_v, h0, conv_tail, ws, L, st);
}

hh_status hh_prefill(const hh_dims *dims, const hh_weights *w, const void *x, int32_t batch,
                     int32_t seqlen, const hh_meta *meta, int32_t window, int32_t is_global,
                     void *out, hh_kv *kv, hh_ssm_state *state, void *ws, size_t ws_bytes,
                     void *stream) {
  Shape s;
  hh_status r = check_prefill_call(dims, w, x, batch, seqlen, meta, window, is_global, out, kv, s);
  if (r != HH_OK) return r;
  PrefillLayout L = prefill_layout(s, batch, seqlen);
  if (!ws || ws_bytes < L.total)
    return fail(HH_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, L.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return s.dtype == HH_BF16
             ? prefill_t<hh::bf16>(s, w, x, batch, seqlen, meta, window, is_global, out, kv, state, ws, L, st)
             : prefill_t<float>(s, w, x, batch, seqlen, meta, window, is_global, out, kv, state, ws, L, st);
}

size_t hh_stage_ssm_workspace_size(const hh_dims *dims, int32_t batch, int32_t seqlen) {
  Shape s;
  if (check_dims(dims, 1, s) != HH_OK || batch <= 0 || seqlen <= 0) return 0;
  return hh::scan_carry_bytes(batch, seqlen, s.D, s.N, nullptr);
}

hh_status hh_stage_attn(const hh_dims *dims, const void *q, const void *k, const void *v,
                        const void *meta_k, const void *meta_v, int32_t batch, int32_t seqlen,
                        int32_t window, int32_t is_global, void *o, void *stream) {
  Shape s;
  hh_status r = check_dims(dims, 1, s);
  if (r != HH_OK) return r;
  if (batch <= 0 || seqlen <= 0) return fail(HH_ERR_INVALID_ARG, "batch and seqlen must be positive");
  if ((long long)batch * seqlen > (1LL << 30)) return fail(HH_ERR_UNSUPPORTED, "batch*seqlen above 2^30 tokens");
  if (!is_global && window < 1) return fail(HH_ERR_INVALID_ARG, "window must be >= 1");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(HH_ERR_INVALID_ARG, "q/k/v/o NULL or not 16-byte aligned");
  if (s.m > 0 && (!aligned16(meta_k) || !aligned16(meta_v)))
    return fail(HH_ERR_INVALID_ARG, "meta k/v NULL or not 16-byte aligned");
  hh::AttnArgs aa{};
  aa.q = q; aa.k = k; aa.v = v; aa.mk = meta_k; aa.mv = meta_v; aa.o = o;
  aa.B = batch; aa.n = seqlen; aa.m = s.m; aa.H = s.H; aa.G = s.G; aa.hd = s.hd;
  aa.window = window; aa.is_global = is_global;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Stage sg(st, "stage_attn");
  const hipError_t err = sg.run([&] {
    return s.dtype == HH_BF16 ? hh::launch_attention<hh::bf16>(aa, st) : hh::launch_attention<float>(aa, st);
  });
  return err == hipSuccess ? HH_OK : hip_fail(err, "attention");
}

hh_status hh_stage_ssm(const hh_dims *dims, const hh_weights *w, const float *xs, const void *z,
                       const float *delta, const float *bc, const float *h0, const float *conv_tail,
                       int32_t batch, int32_t seqlen, void *y, float *h_out, float *tail_out, void *ws,
                       size_t ws_bytes, void *stream) {
  Shape s;
  hh_status r = check_dims(dims, 1, s);
  if (r != HH_OK) return r;
  if (!w || !w->A || !w->conv_w || !w->conv_b) return fail(HH_ERR_INVALID_ARG, "A/conv_w/conv_b NULL");
  if (batch <= 0 || seqlen <= 0) return fail(HH_ERR_INVALID_ARG, "batch and seqlen must be positive");
  if ((long long)batch * seqlen > (1LL << 30)) return fail(HH_ERR_UNSUPPORTED, "batch*seqlen above 2^30 tokens");
  if (!xs || !delta || !bc) return fail(HH_ERR_INVALID_ARG, "xs/delta/bc NULL");
  if (y && !z) return fail(HH_ERR_INVALID_ARG, "y needs the gate z");
  int chunk = 0;
  const size_t need = hh::scan_carry_bytes(batch, seqlen, s.D, s.N, &chunk);
  if (!ws || ws_bytes < need) return fail(HH_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  hh::ScanArgs sa{};
  sa.xs = xs; sa.z = y ? z : nullptr; sa.dt = delta; sa.bc = bc;
  sa.A = w->A; sa.conv_w = w->conv_w; sa.conv_b = w->conv_b;
  sa.h0 = h0; sa.tail0 = conv_tail;
  sa.y = y; sa.h_out = h_out; sa.tail_out = tail_out;
  sa.carry = static_cast<float *>(ws);
  sa.B = batch; sa.n = seqlen; sa.D = s.D; sa.N = s.N; sa.k = s.k; sa.S = s.S; sa.chunk = chunk;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Stage sg(st, "stage_ssm");
  const hipError_t err = sg.run([&] {
    return s.dtype == HH_BF16 ? hh::launch_scan<hh::bf16>(sa, st) : hh::launch_scan<float>(sa, st);
  });
  return err == hipSuccess ? HH_OK : hip_fail(err, "selective scan");
}

hh_status hh_decode_step(const hh_dims *dims, const hh_weights *w, const void *x_t, int32_t batch,
                         const hh_meta *meta, int32_t window, int32_t is_global, hh_kv *kv,
                         hh_ssm_state *state, void *out, void *ws, size_t ws_bytes, void *stream) {
  Shape s;
  hh_status r = check_decode_call(dims, w, x_t, batch, meta, window, is_global, kv, state, out, s);
  if (r != HH_OK) return r;
  DecodeLayout L = decode_layout(s, batch, max_real_keys(kv, window, is_global));
  if (!ws || ws_bytes < L.total)
    return fail(HH_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, L.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return s.dtype == HH_BF16
             ? decode_t<hh::bf16>(s, w, x_t, batch, meta, window, is_global, kv, state, out, ws, L, st)
             : decode_t<float>(s, w, x_t, batch, meta, window, is_global, kv, state, out, ws, L, st);
}

hh_status hh_decode_step_noalloc(const hh_dims *dims, const hh_weights *w, const void *x_t, int32_t batch,
                                 const hh_meta *meta, int32_t window, int32_t is_global, hh_kv *kv,
                                 hh_ssm_state *state, void *out, void *stream) {
  Shape s;
  hh_status r = check_decode_call(dims, w, x_t, batch, meta, window, is_global, kv, state, out, s);
  if (r != HH_OK) return r;
  DecodeLayout L = decode_layout(s, batch, max_real_keys(kv, window, is_global));
  if (L.total > kStaticScratchBytes)
    return fail(HH_ERR_WORKSPACE, "this step needs %zu bytes of scratch; the static scratch holds %zu "
                "(use hh_decode_step with a workspace)", L.total, kStaticScratchBytes);
  void *ws = nullptr;
  if ((r = static_scratch(&ws)) != HH_OK) return r;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return s.dtype == HH_BF16
             ? decode_t<hh::bf16>(s, w, x_t, batch, meta, window, is_global, kv, state, out, ws, L, st)
             : decode_t<float>(s, w, x_t, batch, meta, window, is_global, kv, state, out, ws, L, st);
}

size_t hh_block_meta_prefix_workspace_size(const hh_dims *dims, int32_t kv_producer) {
  Shape s;
  if (!dims || dims->n_meta <= 0 || check_dims(dims, kv_producer, s) != HH_OK) return 0;
  return up256(prefill_layout(s, 1, s.m).total) + (size_t)s.m * s.d * s.es;
}

hh_status hh_block_meta_prefix(const hh_dims *dims, const hh_block_weights *w,
                               const void *meta_tokens, void *meta_k, void *meta_v, float *h0,
                               float *conv_tail, void *ws, size_t ws_bytes, void *stream) {
  hh_status r = check_block_weights(w);
  if (r != HH_OK) return r;
  Shape s;
  if ((r = check_dims(dims, w->mixer.kv_producer, s)) != HH_OK) return r;
  if ((r = check_weights(&w->mixer, s)) != HH_OK) return r;
  if ((r = check_block_shape(w, s)) != HH_OK) return r;
  if (s.m <= 0) return fail(HH_ERR_INVALID_ARG, "n_meta must be positive for hh_block_meta_prefix");
  if (!aligned16(meta_tokens)) return fail(HH_ERR_INVALID_ARG, "meta_tokens NULL or not 16-byte aligned");
  if (s.KV && (!meta_k || !meta_v)) return fail(HH_ERR_INVALID_ARG, "meta_k/meta_v NULL for a producer layer");
  if (!h0 || !conv_tail) return fail(HH_ERR_INVALID_ARG, "h0/conv_tail NULL");
  PrefillLayout L = prefill_layout(s, 1, s.m);
  const size_t off = up256(L.total), need = off + (size_t)s.m * s.d * s.es;
  if (!ws || ws_bytes < need) return fail(HH_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  void *rn = at(ws, off);
  if (s.dtype == HH_BF16) {
    if ((r = block_norm1_t<hh::bf16>(s, w, meta_tokens, s.m, rn, st)) != HH_OK) return r;
    return meta_prefix_t<hh::bf16>(s, &w->mixer, rn, meta_k, meta_v, h0, conv_tail, ws, L, st);
  }
  if ((r = block_norm1_t<float>(s, w, meta_tokens, s.m, rn, st)) != HH_OK) return r;
  return meta_prefix_t<float>(s, &w->mixer, rn, meta_k, meta_v, h0, conv_tail, ws, L, st);
}

size_t hh_block_prefill_workspace_size(const hh_dims *dims, int32_t d_ff, int32_t batch,
                                       int32_t seqlen, int32_t kv_producer) {
  Shape s;
  if (check_dims(dims, kv_producer, s) != HH_OK || batch <= 0 || seqlen <= 0 || d_ff <= 0 ||
      d_ff % (s.dtype == HH_BF16 ? 64 : 4))
    return 0;
  return block_layout(s, prefill_layout(s, batch, seqlen).total, (size_t)batch * seqlen, d_ff).total;
}

hh_status hh_block_prefill(const hh_dims *dims, const hh_block_weights *w, const void *x,
                           int32_t batch, int32_t seqlen, const hh_meta *meta, int32_t window,
                           int32_t is_global, void *out, hh_kv *kv, hh_ssm_state *state, void *ws,
                           size_t ws_bytes, void *stream) {
  hh_status r = check_block_weights(w);
  if (r != HH_OK) return r;
  Shape s;
  r = check_prefill_call(dims, &w->mixer, x, batch, seqlen, meta, window, is_global, out, kv, s);
  if (r != HH_OK) return r;
  if ((r = check_block_shape(w, s)) != HH_OK) return r;
  if (x == out) return fail(HH_ERR_INVALID_ARG, "out must not alias x");
  PrefillLayout L = prefill_layout(s, batch, seqlen);
  BlockLayout BL = block_layout(s, L.total, (size_t)batch * seqlen, w->d_ff);
  if (!ws || ws_bytes < BL.total)
    return fail(HH_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, BL.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return s.dtype == HH_BF16
             ? block_prefill_t<hh::bf16>(s, w, x, batch, seqlen, meta, window, is_global, out, kv, state,
                                         ws, L, BL, st)
             : block_prefill_t<float>(s, w, x, batch, seqlen, meta, window, is_global, out, kv, state, ws,
                                      L, BL, st);
}

size_t hh_block_decode_workspace_size(const hh_dims *dims, int32_t d_ff, int32_t batch, int32_t cap,
                                      int32_t kv_producer) {
  Shape s;
  if (check_dims(dims, kv_producer, s) != HH_OK || batch <= 0 || cap <= 0 || d_ff <= 0 ||
      d_ff % (s.dtype == HH_BF16 ? 64 : 4))
    return 0;
  return block_layout(s, decode_layout(s, batch, cap).total, (size_t)batch, d_ff).total;
}

hh_status hh_block_decode_step(const hh_dims *dims, const hh_block_weights *w, const void *x_t,
                               int32_t batch, const hh_meta *meta, int32_t window, int32_t is_global,
                               hh_kv *kv, hh_ssm_state *state, void *out, void *ws, size_t ws_bytes,
                               void *stream) {
  hh_status r = check_block_weights(w);
  if (r != HH_OK) return r;
  Shape s;
  r = check_decode_call(dims, &w->mixer, x_t, batch, meta, window, is_global, kv, state, out, s);
  if (r != HH_OK) return r;
  if ((r = check_block_shape(w, s)) != HH_OK) return r;
  if (x_t == out) return fail(HH_ERR_INVALID_ARG, "out must not alias x_t");
  DecodeLayout L = decode_layout(s, batch, max_real_keys(kv, window, is_global));
  BlockLayout BL = block_layout(s, L.total, (size_t)batch, w->d_ff);
  if (!ws || ws_bytes < BL.total)
    return fail(HH_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, BL.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return s.dtype == HH_BF16
             ? block_decode_t<hh::bf16>(s, w, x_t, batch, meta, window, is_global, kv, state, out, ws, L,
                                        BL, st)
             : block_decode_t<float>(s, w, x_t, batch, meta, window, is_global, kv, state, out, ws, L, BL,
                                     st);
}

}  // extern "C"
