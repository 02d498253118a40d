// abi.cpp -- C ABI of the sequence-mixer library: argument checks, workspace
// layout, segment plan and dispatch. The kernels live in gma.hip and linattn.hip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <string>
#include <utility>

#include "../../include/linmix.h"
#include "launch.hpp"

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int ok() {
  g_err.clear();
  return LM_OK;
}

constexpr int64_t kChunk = 64;
static_assert(lm::kNoallocScratchBytes == LM_NOALLOC_SCRATCH_BYTES, "scratch size of the header and the library");
// Workgroups the segment plan aims for: one per compute unit of an MI355X.
// Workgroups to aim for when a launch is cut into segments: one per CU for the
// linear-attention kernels, two per CU for the bf16 GMA kernel (it is sized to
// share a CU).
constexpr int64_t kTargetGroups = 256;
constexpr int64_t kTargetGroupsGma = 512;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int64_t P;
  int64_t seg_len;
};

// Cuts each sequence into P segments of whole chunks. An automatic plan
// (segments == 0) makes each segment a multiple of `granule` chunks. Depends
// only on the shapes (and the caller's explicit request), so results are
// reproducible.
Plan plan_segments(int64_t BH, int64_t N, int64_t segments, int64_t target = kTargetGroups, int64_t granule = 1) {
  const int64_t nch = (N + kChunk - 1) / kChunk;
  int64_t P = segments > 0 ? segments : (target + BH - 1) / BH;
  if (P < 1) P = 1;
  if (P > nch) P = nch;
  int64_t cps = (nch + P - 1) / P;
  if (segments == 0) cps = (cps + granule - 1) / granule * granule;
  P = (nch + cps - 1) / cps;
  return Plan{P, cps * kChunk};
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

size_t esize(int dtype) { return dtype == LM_BF16 ? 2 : 4; }

// Carried states: 16-byte aligned, clear of `out` and the workspace, and either
// the same buffer for input and output or two that do not overlap.
int check_states(const char* fn, const float* sin, float* sout, size_t nbytes, const void* out, size_t nout,
                 const void* ws, size_t nws) {
  for (const float* p : {sin, static_cast<const float*>(sout)}) {
    if (!p) continue;
    if (!aligned(p, 16)) return fail(LM_EINVAL, "%s: misaligned state pointer (16 bytes needed)", fn);
    if (overlap(p, nbytes, out, nout) || overlap(p, nbytes, ws, nws))
      return fail(LM_EINVAL, "%s: a state buffer overlaps out or the workspace", fn);
  }
  if (sin && sout && sin != sout && overlap(sin, nbytes, sout, nbytes))
    return fail(LM_EINVAL, "%s: state_in and state_out overlap without being the same buffer", fn);
  return LM_OK;
}

// ----------------------------------------------------------------------------- GMA

// Components are padded to KP (padding has logit -inf). The bf16 kernel for
// d <= 64 works on 64 or 128 components.
bool gma_fast(int64_t d, int64_t K, int dtype) { return dtype == LM_BF16 && d <= 64 && K <= 128; }
// The bf16 kernel for d = 128 and 129..256 components (256 padded).
bool gma_long(int64_t d, int64_t K, int dtype) { return dtype == LM_BF16 && d == 128 && K > 128 && K <= 256; }

int gma_kp(int64_t K, int64_t d, int dtype) {
  if (gma_fast(d, K, dtype)) return K <= 64 ? 64 : 128;
  if (K <= 32) return 32;
  if (K <= 64) return 64;
  if (K <= 128) return 128;
  return 256;
}

struct GmaLayout {
  size_t W, c, agg, aggz, gk, total;  // gk == 0: no key-responsibility buffer
  Plan plan;
  int64_t KP;
};

GmaLayout gma_layout(int64_t B, int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv, int dtype,
                     int64_t segments, int causal, bool store_gk = true) {
  GmaLayout L;
  L.KP = gma_kp(K, d, dtype);
  L.plan = plan_segments(B * H, N, segments, gma_fast(d, K, dtype) ? kTargetGroupsGma : kTargetGroups);
  size_t off = 0;
  L.W = off;
  off = align_up(off + (size_t)H * L.KP * 2 * d * esize(dtype));
  L.c = off;
  off = align_up(off + (size_t)H * L.KP * 4);
  L.agg = off;
  off = align_up(off + (size_t)B * H * L.plan.P * L.KP * dv * 4);
  L.aggz = off;
  off = align_up(off + (size_t)B * H * L.plan.P * L.KP * 4);
  // causal bf16 kernels over several segments: the segment pass stores each
  // chunk's key responsibilities (64 x KP bf16) for the causal pass
  L.gk = 0;
  if (store_gk && causal && (gma_fast(d, K, dtype) || gma_long(d, K, dtype)) && L.plan.P > 1) {
    L.gk = off;
    off = align_up(off + (size_t)B * H * ((N + kChunk - 1) / kChunk) * kChunk * L.KP * 2);
  }
  L.total = off;
  return L;
}

int gma_check_shape(int64_t B, int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv, int causal,
                    int dtype, int64_t segments) {
  if (B < 1 || H < 1 || N < 1 || d < 1 || K < 1 || dv < 1)
    return fail(LM_EINVAL, "sizes must be >= 1 (B=%lld H=%lld N=%lld d=%lld K=%lld dv=%lld)",
                (long long)B, (long long)H, (long long)N, (long long)d, (long long)K, (long long)dv);
  if (dtype != LM_F32 && dtype != LM_BF16) return fail(LM_EINVAL, "dtype %d is not LM_F32 or LM_BF16", dtype);
  if (causal != 0 && causal != 1) return fail(LM_EINVAL, "causal must be 0 or 1 (got %d)", causal);
  if (segments < 0) return fail(LM_EINVAL, "segments must be >= 0 (got %lld)", (long long)segments);
  if (!(d == 32 || d == 64 || d == 128) || dv != d)
    return fail(LM_EUNSUPPORTED, "gma_forward implements d == dv in {32, 64, 128} (got d=%lld dv=%lld)",
                (long long)d, (long long)dv);
  if (K > 256) return fail(LM_EUNSUPPORTED, "gma_forward implements K <= 256 (got %lld)", (long long)K);
  if (dtype == LM_F32 && d == 128 && K > 128)
    return fail(LM_EUNSUPPORTED, "gma_forward in float32 implements K <= 128 at d = 128 (got %lld)", (long long)K);
  if (N > (int64_t(1) << 30) || B * H > 65535)
    return fail(LM_EUNSUPPORTED, "N <= 2^30 and B*H <= 65535 are implemented");
  return LM_OK;
}

// ----------------------------------------------------------------------------- linear attention

// The segment-state pass runs over kLinSub sub-segments per segment: twice the
// workgroups of the chunk pass, two of them sharing a CU.
constexpr int64_t kLinSub = 2;

struct LinLayout {
  size_t agg, total;
  Plan plan;
  int64_t R;
};

LinLayout lin_layout(int64_t B, int64_t H, int64_t N, int64_t dk, bool ccq, int64_t segments) {
  LinLayout L;
  L.plan = plan_segments(B * H, N, segments, kTargetGroups, kLinSub);
  L.R = L.plan.P > 1 && (L.plan.seg_len / kChunk) % kLinSub == 0 ? kLinSub : 1;
  L.agg = 0;
  L.total = align_up((size_t)B * H * L.R * L.plan.P * lm::lin_state_floats(dk, ccq) * 4);
  return L;
}

// allow32: the call also runs with chunks of 32 tokens (the plain and CCQ
// forwards of decayed linear attention).
int lin_check_shape(const char* fn, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                    int dtype, int64_t segments, bool allow32 = false) {
  if (B < 1 || H < 1 || N < 1 || dk < 1 || dv < 1 || chunk < 1)
    return fail(LM_EINVAL, "%s: sizes must be >= 1", fn);
  if (dtype != LM_F32 && dtype != LM_BF16) return fail(LM_EINVAL, "%s: dtype %d is not LM_F32 or LM_BF16", fn, dtype);
  if (segments < 0) return fail(LM_EINVAL, "%s: segments must be >= 0", fn);
  if (chunk != kChunk && !(allow32 && chunk == 32))
    return fail(LM_EUNSUPPORTED, "%s: chunk %lld; %s implemented", fn, (long long)chunk,
                allow32 ? "32 and 64 are" : "64 is");
  if (!(dk == 32 || dk == 64 || dk == 128) || dv != dk)
    return fail(LM_EUNSUPPORTED, "%s implements dk == dv in {32, 64, 128} (got dk=%lld dv=%lld)", fn,
                (long long)dk, (long long)dv);
  if (N > (int64_t(1) << 30) || B * H > 65535)
    return fail(LM_EUNSUPPORTED, "%s: N <= 2^30 and B*H <= 65535 are implemented", fn);
  return LM_OK;
}

int lin_forward(const char* fn, bool ccq, const void* q, const void* k, const void* v, const float* g,
                const float* w_lambda, const float* b_lambda, void* out, int64_t B, int64_t H, int64_t N,
                int64_t dk, int64_t dv, int64_t chunk, int dtype, int64_t segments, int64_t t_in,
                const float* state_in, float* state_out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = lin_check_shape(fn, B, H, N, dk, dv, chunk, dtype, segments, true);
  if (st != LM_OK) return st;
  if (!q || !k || !v || !g || !out || !workspace || (ccq && (!w_lambda || !b_lambda)))
    return fail(LM_EINVAL, "%s: null pointer argument", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(workspace, 16) ||
      !aligned(g, 4) || (ccq && (!aligned(w_lambda, 4) || !aligned(b_lambda, 4))))
    return fail(LM_EINVAL, "%s: misaligned pointer (tensors need 16 bytes, parameters 4)", fn);
  const size_t es = esize(dtype);
  const size_t nq = (size_t)B * H * N * dk * es, nv = (size_t)B * H * N * dv * es;
  const LinLayout L = lin_layout(B, H, N, dk, ccq, segments);
  if (workspace_bytes < L.total)
    return fail(LM_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, L.total);
  if (overlap(out, nv, q, nq) || overlap(out, nv, k, nq) || overlap(out, nv, v, nv) ||
      overlap(out, nv, g, (size_t)B * H * N * 4) || overlap(out, nv, workspace, L.total))
    return fail(LM_EINVAL, "%s: out overlaps an input or the workspace", fn);
  if (t_in < 0 || (t_in > 0 && !state_in) || t_in > (int64_t(1) << 40))
    return fail(LM_EINVAL, "%s: t_in counts the tokens held by state_in (0 without one; got %lld)", fn,
                (long long)t_in);
  const size_t sfl = (size_t)dk * dv + (ccq ? (size_t)dk * dk + dk : 0);
  if ((st = check_states(fn, state_in, state_out, (size_t)B * H * sfl * 4, out, nv, workspace, L.total)) != LM_OK)
    return st;
  lm::LinLaunch La;
  La.q = q;
  La.k = k;
  La.v = v;
  La.g = g;
  La.w_lambda = w_lambda;
  La.b_lambda = b_lambda;
  La.out = out;
  La.agg = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.agg);
  La.B = B;
  La.H = H;
  La.N = N;
  La.D = dk;
  La.P = L.plan.P;
  La.seg_len = L.plan.seg_len;
  La.R = L.R;
  La.bf16 = dtype == LM_BF16;
  La.ccq = ccq;
  La.state_in = state_in;
  La.state_out = state_out;
  La.t_in = t_in;
  La.chunk = chunk;
  hipError_t e = lm::linattn_launch(La, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LM_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

// ----------------------------------------------------------------------------- gated delta rule

struct DeltaLayout {
  size_t w, u, qc, agg, total;
  Plan plan;
};

// W and Ut of every chunk (input dtype, the shapes of K and V); for CCQ also
// the clean queries (input dtype) and the clean-query pass's segment blocks.
DeltaLayout delta_layout(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int dtype, bool ccq,
                         int64_t segments) {
  DeltaLayout L{};
  L.plan = plan_segments(B * H, N, segments);
  const size_t es = esize(dtype);
  L.w = 0;
  L.u = align_up((size_t)B * H * N * dk * es);
  L.total = align_up(L.u + (size_t)B * H * N * dv * es);
  if (!ccq) return L;
  L.qc = L.total;
  L.agg = align_up(L.qc + (size_t)B * H * N * dk * es);
  L.total = align_up(L.agg + (size_t)B * H * L.plan.P * lm::cq_state_floats(dk) * 4);
  return L;
}

int delta_check_shape(const char* fn, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                      int dtype, int64_t segments) {
  int st = lin_check_shape(fn, B, H, N, dk, dv, chunk, dtype, segments);
  if (st != LM_OK) return st;
  if (dtype == LM_F32 && dk > 64)
    return fail(LM_EUNSUPPORTED, "%s implements float32 at dk == dv in {32, 64} (got %lld)", fn, (long long)dk);
  return LM_OK;
}

int delta_forward(const char* fn, bool ccq, const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* w_lambda, const float* b_lambda, void* out, int64_t B, int64_t H,
                  int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype, int64_t segments, int64_t t_in,
                  const float* state_in, float* state_out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = delta_check_shape(fn, B, H, N, dk, dv, chunk, dtype, segments);
  if (st != LM_OK) return st;
  const DeltaLayout L = delta_layout(B, H, N, dk, dv, dtype, ccq, segments);
  if (!q || !k || !v || !g || !beta || !out || !workspace || (ccq && (!w_lambda || !b_lambda)))
    return fail(LM_EINVAL, "%s: null pointer argument", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(workspace, 16) ||
      !aligned(g, 4) || !aligned(beta, 4) || (ccq && (!aligned(w_lambda, 4) || !aligned(b_lambda, 4))))
    return fail(LM_EINVAL, "%s: misaligned pointer (tensors need 16 bytes, parameters 4)", fn);
  if (workspace_bytes < L.total)
    return fail(LM_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, L.total);
  const size_t es = esize(dtype);
  const size_t nq = (size_t)B * H * N * dk * es, nv = (size_t)B * H * N * dv * es, nt = (size_t)B * H * N * 4;
  if (overlap(out, nv, q, nq) || overlap(out, nv, k, nq) || overlap(out, nv, v, nv) || overlap(out, nv, g, nt) ||
      overlap(out, nv, beta, nt) || overlap(out, nv, workspace, L.total))
    return fail(LM_EINVAL, "%s: out overlaps an input or the workspace", fn);
  if (t_in < 0 || (t_in > 0 && !state_in) || t_in > (int64_t(1) << 40))
    return fail(LM_EINVAL, "%s: t_in counts the tokens held by state_in (0 without one; got %lld)", fn,
                (long long)t_in);
  const size_t sfl = (size_t)dk * dv + (ccq ? (size_t)dk * dk + dk : 0);
  if ((st = check_states(fn, state_in, state_out, (size_t)B * H * sfl * 4, out, nv, workspace, L.total)) != LM_OK)
    return st;
  lm::DeltaLaunch La{};
  La.q = q;
  La.k = k;
  La.v = v;
  La.g = g;
  La.beta = beta;
  La.w_lambda = w_lambda;
  La.b_lambda = b_lambda;
  La.out = out;
  La.wbuf = static_cast<char*>(workspace) + L.w;
  La.ubuf = static_cast<char*>(workspace) + L.u;
  La.qc = ccq ? static_cast<char*>(workspace) + L.qc : nullptr;
  La.agg = ccq ? reinterpret_cast<float*>(static_cast<char*>(workspace) + L.agg) : nullptr;
  La.B = B;
  La.H = H;
  La.N = N;
  La.D = dk;
  La.dv = dv;
  La.P = L.plan.P;
  La.seg_len = L.plan.seg_len;
  La.bf16 = dtype == LM_BF16;
  La.ccq = ccq;
  La.state_in = state_in;
  La.state_out = state_out;
  La.sstride = (int64_t)sfl;
  La.t_in = t_in;
  hipError_t e = lm::deltanet_launch(La, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LM_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

struct VecLayout {
  size_t total;
  Plan plan;
  int64_t R;
};

// Same plan as the scalar-gate form: segments of whole chunks, the segment pass
// over two sub-segments per segment when the segment length is an even number
// of chunks.
VecLayout vec_layout(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t segments) {
  VecLayout L;
  L.plan = plan_segments(B * H, N, segments, kTargetGroups, kLinSub);
  L.R = L.plan.P > 1 && (L.plan.seg_len / kChunk) % kLinSub == 0 ? kLinSub : 1;
  L.total = align_up((size_t)B * H * L.R * L.plan.P * lm::vec_state_floats(dk) * 4);
  return L;
}

int gma_impl(const char* fn, const void* q, const void* k, const void* v, const float* mu, const float* log_var,
             const float* logit_pi, void* out, int64_t B, int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv,
             int causal, float eps, int dtype, int64_t segments, const float* state_in, float* state_out,
             void* workspace, size_t workspace_bytes, void* stream, bool store_gk = true) {
  int st = gma_check_shape(B, H, N, d, K, dv, causal, dtype, segments);
  if (st != LM_OK) return st;
  if (!(eps >= 0.f) || std::isinf(eps)) return fail(LM_EINVAL, "%s: eps must be finite and >= 0", fn);
  if (!q || !k || !v || !mu || !log_var || !logit_pi || !out || !workspace)
    return fail(LM_EINVAL, "%s: null pointer argument", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(workspace, 16) ||
      !aligned(mu, 4) || !aligned(log_var, 4) || !aligned(logit_pi, 4))
    return fail(LM_EINVAL, "%s: misaligned pointer (tensors need 16 bytes, parameters 4)", fn);
  const GmaLayout L = gma_layout(B, H, N, d, K, dv, dtype, segments, causal, store_gk);
  if (workspace_bytes < L.total)
    return fail(LM_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, L.total);
  const size_t es = esize(dtype);
  const size_t nq = (size_t)B * H * N * d * es, nv = (size_t)B * H * N * dv * es;
  if (overlap(out, nv, q, nq) || overlap(out, nv, k, nq) || overlap(out, nv, v, nv) ||
      overlap(out, nv, workspace, L.total) || overlap(out, nv, mu, (size_t)H * K * d * 4) ||
      overlap(out, nv, log_var, (size_t)H * K * d * 4) || overlap(out, nv, logit_pi, (size_t)H * K * 4))
    return fail(LM_EINVAL, "%s: out overlaps an input or the workspace", fn);
  if ((st = check_states(fn, state_in, state_out, (size_t)B * H * (K * dv + K) * 4, out, nv, workspace,
                         L.total)) != LM_OK)
    return st;
  lm::GmaLaunch La;
  char* ws = static_cast<char*>(workspace);
  La.q = q;
  La.k = k;
  La.v = v;
  La.out = out;
  La.mu = mu;
  La.log_var = log_var;
  La.logit_pi = logit_pi;
  La.W = ws + L.W;
  La.c = reinterpret_cast<float*>(ws + L.c);
  La.agg = reinterpret_cast<float*>(ws + L.agg);
  La.aggz = reinterpret_cast<float*>(ws + L.aggz);
  La.gk = L.gk ? ws + L.gk : nullptr;
  La.B = B;
  La.H = H;
  La.N = N;
  La.D = d;
  La.K = K;
  La.KP = L.KP;
  La.P = L.plan.P;
  La.seg_len = L.plan.seg_len;
  La.causal = causal;
  La.bf16 = dtype == LM_BF16;
  La.eps = eps;
  La.state_in = state_in;
  La.state_out = state_out;
  hipError_t e = lm::gma_launch(La, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LM_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

// One-token steps: shapes as the forwards with N = 1, state in place.
int dec_check(const char* fn, int64_t B, int64_t H, int64_t d, int64_t dv, int dtype) {
  if (B < 1 || H < 1 || d < 1 || dv < 1) return fail(LM_EINVAL, "%s: sizes must be >= 1", fn);
  if (dtype != LM_F32 && dtype != LM_BF16) return fail(LM_EINVAL, "%s: dtype %d is not LM_F32 or LM_BF16", fn, dtype);
  if (!(d == 32 || d == 64 || d == 128) || dv != d)
    return fail(LM_EUNSUPPORTED, "%s implements d == dv in {32, 64, 128} (got %lld, %lld)", fn, (long long)d,
                (long long)dv);
  if (B * H > (int64_t(1) << 24)) return fail(LM_EUNSUPPORTED, "%s: B*H <= 2^24 is implemented", fn);
  return LM_OK;
}

int dec_run(const char* fn, bool gma, bool ccq, lm::DecodeLaunch& La, int64_t d, size_t state_floats,
            void* stream) {
  const size_t es = La.bf16 ? 2 : 4;
  const size_t nx = (size_t)La.B * La.H * d * es, ns = (size_t)La.B * La.H * state_floats * 4;
  if (!La.q || !La.k || !La.v || !La.out || !La.state) return fail(LM_EINVAL, "%s: null pointer argument", fn);
  if (!aligned(La.q, 16) || !aligned(La.k, 16) || !aligned(La.v, 16) || !aligned(La.out, 16) ||
      !aligned(La.state, 16))
    return fail(LM_EINVAL, "%s: misaligned pointer (tensors and the state need 16 bytes)", fn);
  if (overlap(La.out, nx, La.q, nx) || overlap(La.out, nx, La.k, nx) || overlap(La.out, nx, La.v, nx) ||
      overlap(La.out, nx, La.state, ns))
    return fail(LM_EINVAL, "%s: out overlaps an input or the state", fn);
  if (overlap(La.state, ns, La.q, nx) || overlap(La.state, ns, La.k, nx) || overlap(La.state, ns, La.v, nx))
    return fail(LM_EINVAL, "%s: the state overlaps an input", fn);
  hipError_t e = gma ? lm::gma_decode_launch(La, static_cast<hipStream_t>(stream))
                     : lm::lin_decode_launch(La, ccq, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LM_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

int vec_forward(const char* fn, const void* q, const void* k, const void* v, const float* g, void* out, int64_t B,
                int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype, int64_t segments,
                const float* state_in, float* state_out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = lin_check_shape(fn, B, H, N, dk, dv, chunk, dtype, segments);
  if (st != LM_OK) return st;
  if (!q || !k || !v || !g || !out || !workspace) return fail(LM_EINVAL, "%s: null pointer argument", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) || !aligned(out, 16) ||
      !aligned(workspace, 16))
    return fail(LM_EINVAL, "%s: misaligned pointer (16 bytes needed)", fn);
  const size_t es = esize(dtype);
  const size_t nq = (size_t)B * H * N * dk * es, nv = (size_t)B * H * N * dv * es, ng = (size_t)B * H * N * dk * 4;
  const VecLayout L = vec_layout(B, H, N, dk, segments);
  if (workspace_bytes < L.total)
    return fail(LM_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, L.total);
  if (overlap(out, nv, q, nq) || overlap(out, nv, k, nq) || overlap(out, nv, v, nv) || overlap(out, nv, g, ng) ||
      overlap(out, nv, workspace, L.total))
    return fail(LM_EINVAL, "%s: out overlaps an input or the workspace", fn);
  if ((st = check_states(fn, state_in, state_out, (size_t)B * H * dk * dv * 4, out, nv, workspace, L.total)) != LM_OK)
    return st;
  lm::VecLaunch La;
  La.q = q;
  La.k = k;
  La.v = v;
  La.g = g;
  La.out = out;
  La.agg = static_cast<float*>(workspace);
  La.B = B;
  La.H = H;
  La.N = N;
  La.D = dk;
  La.P = L.plan.P;
  La.seg_len = L.plan.seg_len;
  La.R = L.R;
  La.bf16 = dtype == LM_BF16;
  La.state_in = state_in;
  La.state_out = state_out;
  hipError_t e = lm::linattn_vec_launch(La, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LM_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

// ----------------------------------------------------------------------------- GMA backward

// Width of the inner linear attention of the GMA backward: features are the K
// responsibilities, values [v | 1].
int64_t gma_bwd_width(int64_t K, int64_t dv) {
  const int64_t need = K > dv + 1 ? K : dv + 1;
  return need <= 32 ? 32 : need <= 64 ? 64 : 128;
}

struct GmaBwdLayout {
  size_t iv, cst, rows[8], ones, inner[5], rg, agg, part, sums, tmp[3], total;
  LinLayout lin;
  int64_t DL, nseg, seg_len, NN;
  int64_t NF, NVB;  // wide shapes: blocks of 128 responsibility / value columns (1 otherwise)
  bool wide;
};

// d = 128 or more than 128 components: the inner tensors in blocks of 128 columns.
bool gma_bwd_wide(int64_t d, int64_t K) { return d > 64 || K > 128; }

GmaBwdLayout gma_bwd_layout(int64_t B, int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv, int causal) {
  GmaBwdLayout L;
  L.wide = gma_bwd_wide(d, K);
  L.DL = L.wide ? 128 : gma_bwd_width(K, dv);
  L.NF = L.wide ? (K + 127) / 128 : 1;
  L.NVB = L.wide ? (dv + 128) / 128 : 1;
  L.NN = causal ? N : 2 * N;  // bidirectional: keys in rows [0, N), queries in [N, 2N)
  // token ranges of the routing and chain-rule kernels: about 1024 workgroups
  const int64_t want = (1024 + 2 * B * H - 1) / (2 * B * H);
  int64_t len = (N + want - 1) / want;
  len = (len + 15) / 16 * 16;
  L.seg_len = len;
  L.nseg = (N + len - 1) / len;
  L.lin = lin_layout(B, H, L.NN, L.DL, false, 0);
  // wide: every row tensor holds two blocks (also B*H*N rows of 256 floats)
  const size_t blk = align_up((size_t)B * H * L.NN * L.DL * 4);
  const size_t rowt = L.wide ? 2 * blk : blk, colt = align_up((size_t)B * H * L.NN * 4);
  size_t off = 0;
  L.iv = off;
  off = align_up(off + (size_t)H * K * d * 4);
  L.cst = off;
  off = align_up(off + (size_t)H * K * 4);
  for (int i = 0; i < 8; ++i) {
    L.rows[i] = off;
    off += rowt;
  }
  L.ones = off;
  off += colt;
  for (int i = 0; i < 5; ++i) {
    L.inner[i] = off;
    off += rowt;
  }
  L.rg = off;
  off += colt;
  L.agg = off;
  off += L.lin.total;
  L.part = off;
  off = align_up(off + (size_t)H * 2 * B * L.nseg * K * (2 * d + 1) * 4);
  L.sums = off;
  off = align_up(off + (size_t)H * K * (2 * d + 1) * 4);
  for (int i = 0; i < 3; ++i) {
    L.tmp[i] = off;
    off += L.wide ? blk : 0;
  }
  L.total = off;
  return L;
}

int gma_bwd_check(const char* fn, int64_t B, int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv, int causal,
                  float eps, int dtype) {
  if (B < 1 || H < 1 || N < 1 || d < 1 || K < 1 || dv < 1) return fail(LM_EINVAL, "%s: sizes must be >= 1", fn);
  if (dtype != LM_F32 && dtype != LM_BF16) return fail(LM_EINVAL, "%s: dtype %d is not LM_F32 or LM_BF16", fn, dtype);
  if (causal != 0 && causal != 1) return fail(LM_EINVAL, "%s: causal must be 0 or 1 (got %d)", fn, causal);
  if (!(eps >= 0.f) || std::isinf(eps)) return fail(LM_EINVAL, "%s: eps must be finite and >= 0", fn);
  if (!(d == 32 || d == 64 || d == 128) || dv != d)
    return fail(LM_EUNSUPPORTED, "%s implements d == dv in {32, 64, 128} (got d=%lld dv=%lld)", fn, (long long)d,
                (long long)dv);
  if (K > 256) return fail(LM_EUNSUPPORTED, "%s implements K <= 256 (got %lld)", fn, (long long)K);
  if (N > (int64_t(1) << 29) || B * H > 65535) return fail(LM_EUNSUPPORTED, "%s: N <= 2^29 and B*H <= 65535", fn);
  return LM_OK;
}

// ----------------------------------------------------------------------------- CCQ backward

struct CcqBwdLayout {
  size_t rows[24], cols[3], csum, part, agg, total;
  int nrows;
  LinLayout lin;
  int64_t nch, clen, nblk, blen;
};

CcqBwdLayout ccq_bwd_layout(int64_t B, int64_t H, int64_t N, int64_t D, int dtype) {
  CcqBwdLayout L;
  L.lin = lin_layout(B, H, N, D, false, 0);
  L.nch = N < 64 ? N : 64;
  L.clen = (N + L.nch - 1) / L.nch;
  L.nch = (N + L.clen - 1) / L.clen;
  int64_t blen = (N * B * H + 1023) / 1024;
  blen = blen < 4 ? 4 : (blen + 3) / 4 * 4;
  L.blen = blen;
  L.nblk = (N + blen - 1) / blen;
  // 13 rows always, 3 input copies and dv for bf16, 5 reversal buffers
  L.nrows = 13 + 5 + (dtype == LM_BF16 ? 4 : 0);
  const size_t rowt = align_up((size_t)B * H * N * D * 4), colt = align_up((size_t)B * H * N * 4);
  size_t off = 0;
  for (int i = 0; i < L.nrows; ++i) {
    L.rows[i] = off;
    off += rowt;
  }
  for (int i = 0; i < 3; ++i) {
    L.cols[i] = off;
    off += colt;
  }
  L.csum = off;
  off = align_up(off + (size_t)B * H * L.nch * D * 4);
  L.part = off;
  off = align_up(off + (size_t)H * B * L.nblk * (D + 1) * 4);
  L.agg = off;
  off += L.lin.total;
  L.total = off;
  return L;
}

// ----------------------------------------------------------------------------- padded shapes
//
// Feature widths of 16, and d != dv, run on the kernels of width D (the
// smallest of 32, 64, 128 that holds both) after zero padding of the feature
// axis (pad.hip; exact, see there). The padded tensors and the output sit in
// the workspace ahead of the inner call's own workspace. Stateless forwards
// only: carried states, decode steps, backward passes and the entry point that
// allocates nothing take the native shapes (d == dv in {32, 64, 128}).

bool width_ok(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool native_widths(int64_t d, int64_t dv) { return d == dv && d != 16; }
int64_t pad_width(int64_t d, int64_t dv) {
  const int64_t m = d > dv ? d : dv;
  return m <= 32 ? 32 : m <= 64 ? 64 : 128;
}

int pad_check(const char* fn, int64_t d, int64_t dv) {
  if (d < 1 || dv < 1) return fail(LM_EINVAL, "%s: sizes must be >= 1", fn);
  if (!width_ok(d) || !width_ok(dv))
    return fail(LM_EUNSUPPORTED, "%s implements feature widths in {16, 32, 64, 128} (got %lld and %lld)", fn,
                (long long)d, (long long)dv);
  return LM_OK;
}

struct PadLayout {
  int64_t D;
  size_t q, k, v, out, g, w, mu, lv, inner, total;
};

// q, k [.., d] -> [.., D]; v [.., dv] -> [.., D]; the output [.., D]; optional
// per-feature decays [.., D] (vec), gate weights [H, D] (w) or routing
// parameters [H, K, D] (mu, log_var; K > 0); then `inner` bytes.
PadLayout pad_layout(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, int dtype, bool vec, bool w, int64_t K,
                     size_t inner) {
  PadLayout L{};
  L.D = pad_width(d, dv);
  const size_t rows = (size_t)B * H * N, es = esize(dtype), t = align_up(rows * L.D * es);
  size_t off = 0;
  L.q = off;
  off += t;
  L.k = off;
  off += t;
  L.v = off;
  off += t;
  L.out = off;
  off += t;
  L.g = off;
  if (vec) off += align_up(rows * L.D * 4);
  L.w = off;
  if (w) off += align_up((size_t)H * L.D * 4);
  L.mu = off;
  if (K) off += align_up((size_t)H * K * L.D * 4);
  L.lv = off;
  if (K) off += align_up((size_t)H * K * L.D * 4);
  L.inner = off;
  L.total = align_up(off + inner);
  return L;
}

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// The caller's pointers of a padded call: null, alignment, and out against the
// inputs and the workspace.
int pad_args(const char* fn, std::initializer_list<const void*> need, const void* out, size_t nout,
             std::initializer_list<std::pair<const void*, size_t>> inputs, const void* ws, size_t nws) {
  for (const void* p : need)
    if (!p) return fail(LM_EINVAL, "%s: null pointer argument", fn);
  if (!out || !ws) return fail(LM_EINVAL, "%s: null pointer argument", fn);
  if (!aligned(out, 16) || !aligned(ws, 16)) return fail(LM_EINVAL, "%s: misaligned out or workspace", fn);
  for (const auto& in : inputs) {
    if (!aligned(in.first, 4)) return fail(LM_EINVAL, "%s: misaligned pointer", fn);
    if (overlap(out, nout, in.first, in.second)) return fail(LM_EINVAL, "%s: out overlaps an input", fn);
    if (overlap(ws, nws, in.first, in.second)) return fail(LM_EINVAL, "%s: an input overlaps the workspace", fn);
  }
  if (overlap(out, nout, ws, nws)) return fail(LM_EINVAL, "%s: out overlaps the workspace", fn);
  return LM_OK;
}

int hip_fail(const char* fn, hipError_t e) { return fail(LM_EHIP, "%s: %s", fn, hipGetErrorString(e)); }

int gma_padded(const char* fn, const void* q, const void* k, const void* v, const float* mu, const float* log_var,
               const float* logit_pi, void* out, int64_t B, int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv,
               int causal, float eps, int dtype, int64_t segments, void* workspace, size_t workspace_bytes,
               void* stream) {
  int st = pad_check(fn, d, dv);
  if (st != LM_OK) return st;
  const int64_t D = pad_width(d, dv);
  if ((st = gma_check_shape(B, H, N, D, K, D, causal, dtype, segments)) != LM_OK) return st;
  if (!(eps >= 0.f) || std::isinf(eps)) return fail(LM_EINVAL, "%s: eps must be finite and >= 0", fn);
  const PadLayout L = pad_layout(B, H, N, d, dv, dtype, false, false, K,
                                 gma_layout(B, H, N, D, K, D, dtype, segments, causal).total);
  const size_t es = esize(dtype), rows = (size_t)B * H * N;
  if ((st = pad_args(fn, {q, k, v, mu, log_var, logit_pi}, out, rows * dv * es,
                     {{q, rows * d * es}, {k, rows * d * es}, {v, rows * dv * es}, {mu, (size_t)H * K * d * 4},
                      {log_var, (size_t)H * K * d * 4}, {logit_pi, (size_t)H * K * 4}},
                     workspace, L.total)) != LM_OK)
    return st;
  if (workspace_bytes < L.total)
    return fail(LM_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, L.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if ((e = lm::pad_cols(q, at(workspace, L.q), rows, (int)d, (int)D, 0.f, (int)es, s)) != hipSuccess ||
      (e = lm::pad_cols(k, at(workspace, L.k), rows, (int)d, (int)D, 0.f, (int)es, s)) != hipSuccess ||
      (e = lm::pad_cols(v, at(workspace, L.v), rows, (int)dv, (int)D, 0.f, (int)es, s)) != hipSuccess ||
      (e = lm::pad_cols(mu, at(workspace, L.mu), H * K, (int)d, (int)D, 0.f, 4, s)) != hipSuccess ||
      (e = lm::pad_cols(log_var, at(workspace, L.lv), H * K, (int)d, (int)D, 0.f, 4, s)) != hipSuccess)
    return hip_fail(fn, e);
  if ((st = gma_impl(fn, at(workspace, L.q), at(workspace, L.k), at(workspace, L.v),
                     reinterpret_cast<const float*>(at(workspace, L.mu)),
                     reinterpret_cast<const float*>(at(workspace, L.lv)), logit_pi, at(workspace, L.out), B, H, N, D,
                     K, D, causal, eps, dtype, segments, nullptr, nullptr, at(workspace, L.inner),
                     L.total - L.inner, stream)) != LM_OK)
    return st;
  if ((e = lm::crop_cols(at(workspace, L.out), out, rows, (int)D, (int)dv, (int)es, s)) != hipSuccess)
    return hip_fail(fn, e);
  return ok();
}

// Linear attention, CCQ, the per-feature decay and the delta rule.
enum class Lin { gla, ccq, vec, delta, ccq_delta };

size_t lin_inner_bytes(Lin kind, int64_t B, int64_t H, int64_t N, int64_t D, int dtype, int64_t segments) {
  switch (kind) {
    case Lin::gla: return lin_layout(B, H, N, D, false, segments).total;
    case Lin::ccq: return lin_layout(B, H, N, D, true, segments).total;
    case Lin::vec: return vec_layout(B, H, N, D, segments).total;
    case Lin::delta: return delta_layout(B, H, N, D, D, dtype, false, segments).total;
    case Lin::ccq_delta: return delta_layout(B, H, N, D, D, dtype, true, segments).total;
  }
  return 0;
}

int lin_pad_check(const char* fn, Lin kind, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                  int dtype, int64_t segments) {
  int st = pad_check(fn, dk, dv);
  if (st != LM_OK) return st;
  const int64_t D = pad_width(dk, dv);
  if (kind == Lin::delta || kind == Lin::ccq_delta) return delta_check_shape(fn, B, H, N, D, D, chunk, dtype, segments);
  return lin_check_shape(fn, B, H, N, D, D, chunk, dtype, segments, kind == Lin::gla || kind == Lin::ccq);
}

PadLayout lin_pad_layout(Lin kind, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int dtype,
                         int64_t segments) {
  const int64_t D = pad_width(dk, dv);
  const bool w = kind == Lin::ccq || kind == Lin::ccq_delta;
  return pad_layout(B, H, N, dk, dv, dtype, kind == Lin::vec, w, 0, lin_inner_bytes(kind, B, H, N, D, dtype, segments));
}

int lin_padded(const char* fn, Lin kind, const void* q, const void* k, const void* v, const float* g,
               const float* beta, const float* w_lambda, const float* b_lambda, void* out, int64_t B, int64_t H,
               int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype, int64_t segments, void* workspace,
               size_t workspace_bytes, void* stream) {
  int st = lin_pad_check(fn, kind, B, H, N, dk, dv, chunk, dtype, segments);
  if (st != LM_OK) return st;
  const bool ccq = kind == Lin::ccq || kind == Lin::ccq_delta, delta = kind == Lin::delta || kind == Lin::ccq_delta;
  const int64_t D = pad_width(dk, dv);
  const PadLayout L = lin_pad_layout(kind, B, H, N, dk, dv, dtype, segments);
  const size_t es = esize(dtype), rows = (size_t)B * H * N;
  const size_t ng = kind == Lin::vec ? rows * dk * 4 : rows * 4;
  if ((st = pad_args(fn, {q, k, v, g, delta ? beta : q, ccq ? w_lambda : q, ccq ? b_lambda : q}, out, rows * dv * es,
                     {{q, rows * dk * es}, {k, rows * dk * es}, {v, rows * dv * es}, {g, ng},
                      {delta ? beta : g, delta ? rows * 4 : 0}, {ccq ? w_lambda : g, ccq ? (size_t)H * dk * 4 : 0},
                      {ccq ? b_lambda : g, ccq ? (size_t)H * 4 : 0}},
                     workspace, L.total)) != LM_OK)
    return st;
  if (workspace_bytes < L.total)
    return fail(LM_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, L.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if ((e = lm::pad_cols(q, at(workspace, L.q), rows, (int)dk, (int)D, 0.f, (int)es, s)) != hipSuccess ||
      (e = lm::pad_cols(k, at(workspace, L.k), rows, (int)dk, (int)D, 0.f, (int)es, s)) != hipSuccess ||
      (e = lm::pad_cols(v, at(workspace, L.v), rows, (int)dv, (int)D, 0.f, (int)es, s)) != hipSuccess)
    return hip_fail(fn, e);
  if (kind == Lin::vec && (e = lm::pad_cols(g, at(workspace, L.g), rows, (int)dk, (int)D, 1.f, 4, s)) != hipSuccess)
    return hip_fail(fn, e);
  if (ccq && (e = lm::pad_cols(w_lambda, at(workspace, L.w), H, (int)dk, (int)D, 0.f, 4, s)) != hipSuccess)
    return hip_fail(fn, e);
  const void *pq = at(workspace, L.q), *pk = at(workspace, L.k), *pv = at(workspace, L.v);
  const float* pw = reinterpret_cast<const float*>(at(workspace, L.w));
  void* po = at(workspace, L.out);
  void* iw = at(workspace, L.inner);
  const size_t nb = L.total - L.inner;
  switch (kind) {
    case Lin::gla:
    case Lin::ccq:
      st = lin_forward(fn, ccq, pq, pk, pv, g, ccq ? pw : nullptr, b_lambda, po, B, H, N, D, D, chunk, dtype, segments,
                       0, nullptr, nullptr, iw, nb, stream);
      break;
    case Lin::vec:
      st = vec_forward(fn, pq, pk, pv, reinterpret_cast<const float*>(at(workspace, L.g)), po, B, H, N, D, D, chunk,
                       dtype, segments, nullptr, nullptr, iw, nb, stream);
      break;
    case Lin::delta:
    case Lin::ccq_delta:
      st = delta_forward(fn, ccq, pq, pk, pv, g, beta, ccq ? pw : nullptr, b_lambda, po, B, H, N, D, D, chunk, dtype,
                         segments, 0, nullptr, nullptr, iw, nb, stream);
      break;
  }
  if (st != LM_OK) return st;
  if ((e = lm::crop_cols(po, out, rows, (int)D, (int)dv, (int)es, s)) != hipSuccess) return hip_fail(fn, e);
  return ok();
}

size_t lin_padded_bytes(const char* fn, Lin kind, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                        int64_t chunk, int dtype, int64_t segments) {
  if (lin_pad_check(fn, kind, B, H, N, dk, dv, chunk, dtype, segments) != LM_OK) return 0;
  return lin_pad_layout(kind, B, H, N, dk, dv, dtype, segments).total;
}

}  // namespace

extern "C" {

int lm_abi_version(void) { return LM_ABI_VERSION; }

const char* lm_status_string(int status) {
  switch (status) {
    case LM_OK: return "LM_OK";
    case LM_EINVAL: return "LM_EINVAL";
    case LM_EUNSUPPORTED: return "LM_EUNSUPPORTED";
    case LM_EWORKSPACE: return "LM_EWORKSPACE";
    case LM_EHIP: return "LM_EHIP";
    default: return "LM_UNKNOWN";
  }
}

const char* lm_last_error(void) { return g_err.c_str(); }

size_t gma_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv, int causal,
                           int dtype, int64_t segments) {
  if (!native_widths(d, dv)) {
    if (pad_check("gma_forward", d, dv) != LM_OK) return 0;
    const int64_t D = pad_width(d, dv);
    if (gma_check_shape(B, H, N, D, K, D, causal, dtype, segments) != LM_OK) return 0;
    return pad_layout(B, H, N, d, dv, dtype, false, false, K, gma_layout(B, H, N, D, K, D, dtype, segments, causal).total)
        .total;
  }
  if (gma_check_shape(B, H, N, d, K, dv, causal, dtype, segments) != LM_OK) return 0;
  return gma_layout(B, H, N, d, K, dv, dtype, segments, causal).total;
}

int gma_forward(const void* q, const void* k, const void* v, const float* mu, const float* log_var,
                const float* logit_pi, void* out, int64_t B, int64_t H, int64_t N, int64_t d, int64_t K,
                int64_t dv, int causal, float eps, int dtype, int64_t segments, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (!native_widths(d, dv))
    return gma_padded("gma_forward", q, k, v, mu, log_var, logit_pi, out, B, H, N, d, K, dv, causal, eps, dtype,
                      segments, workspace, workspace_bytes, stream);
  return gma_impl("gma_forward", q, k, v, mu, log_var, logit_pi, out, B, H, N, d, K, dv, causal, eps, dtype,
                  segments, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int gma_forward_noalloc(const void* q, const void* k, const void* v, const float* mu, const float* log_var,
                        const float* logit_pi, void* out, int64_t B, int64_t H, int64_t N, int64_t d, int64_t K,
                        int64_t dv, int causal, float eps, int dtype, int64_t segments, void* stream) {
  const char* fn = "gma_forward_noalloc";
  int st = gma_check_shape(B, H, N, d, K, dv, causal, dtype, segments);
  if (st != LM_OK) return st;
  // (every argument is checked before the first HIP call, as for gma_forward)
  if (!(eps >= 0.f) || std::isinf(eps)) return fail(LM_EINVAL, "%s: eps must be finite and >= 0", fn);
  if (!q || !k || !v || !mu || !log_var || !logit_pi || !out) return fail(LM_EINVAL, "%s: null pointer argument", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(mu, 4) ||
      !aligned(log_var, 4) || !aligned(logit_pi, 4))
    return fail(LM_EINVAL, "%s: misaligned pointer (tensors need 16 bytes, parameters 4)", fn);
  // the fixed scratch never holds the stored key responsibilities
  const size_t need = gma_layout(B, H, N, d, K, dv, dtype, segments, causal, false).total;
  if (need > lm::kNoallocScratchBytes)
    return fail(LM_EWORKSPACE, "%s: %zu bytes of scratch needed, the fixed scratch holds %zu", fn, need,
                lm::kNoallocScratchBytes);
  void* ws = nullptr;
  const hipError_t e = lm::noalloc_scratch(&ws);
  if (e != hipSuccess) return fail(LM_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return gma_impl(fn, q, k, v, mu, log_var, logit_pi, out, B, H, N, d, K, dv, causal, eps, dtype, segments,
                  nullptr, nullptr, ws, lm::kNoallocScratchBytes, stream, false);
}

int gma_forward_state(const void* q, const void* k, const void* v, const float* mu, const float* log_var,
                      const float* logit_pi, void* out, int64_t B, int64_t H, int64_t N, int64_t d, int64_t K,
                      int64_t dv, float eps, int dtype, int64_t segments, const float* state_in,
                      float* state_out, void* workspace, size_t workspace_bytes, void* stream) {
  return gma_impl("gma_forward_state", q, k, v, mu, log_var, logit_pi, out, B, H, N, d, K, dv, 1, eps, dtype,
                  segments, state_in, state_out, workspace, workspace_bytes, stream);
}

int gma_decode_step(const void* q, const void* k, const void* v, const float* mu, const float* log_var,
                    const float* logit_pi, void* out, float* state, int64_t B, int64_t H, int64_t d, int64_t K,
                    int64_t dv, float eps, int dtype, void* stream) {
  const char* fn = "gma_decode_step";
  int st = dec_check(fn, B, H, d, dv, dtype);
  if (st != LM_OK) return st;
  if (K < 1 || K > 256) return fail(K < 1 ? LM_EINVAL : LM_EUNSUPPORTED, "%s: 1 <= K <= 256 (got %lld)", fn,
                                    (long long)K);
  if (!(eps >= 0.f) || std::isinf(eps)) return fail(LM_EINVAL, "%s: eps must be finite and >= 0", fn);
  if (!mu || !log_var || !logit_pi) return fail(LM_EINVAL, "%s: null pointer argument", fn);
  if (!aligned(mu, 4) || !aligned(log_var, 4) || !aligned(logit_pi, 4))
    return fail(LM_EINVAL, "%s: misaligned parameter pointer", fn);
  lm::DecodeLaunch La{};
  La.q = q;
  La.k = k;
  La.v = v;
  La.mu = mu;
  La.log_var = log_var;
  La.logit_pi = logit_pi;
  La.out = out;
  La.state = state;
  La.B = B;
  La.H = H;
  La.D = d;
  La.K = K;
  La.bf16 = dtype == LM_BF16;
  La.eps = eps;
  return dec_run(fn, true, false, La, d, (size_t)K * dv + K, stream);
}

size_t linattn_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype,
                               int64_t segments) {
  if (!native_widths(dk, dv))
    return lin_padded_bytes("linattn_chunk_forward", Lin::gla, B, H, N, dk, dv, chunk, dtype, segments);
  if (lin_check_shape("linattn_chunk_forward", B, H, N, dk, dv, chunk, dtype, segments, true) != LM_OK) return 0;
  return lin_layout(B, H, N, dk, false, segments).total;
}

int linattn_chunk_forward(const void* q, const void* k, const void* v, const float* g, void* out, int64_t B,
                          int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype, int64_t segments,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!native_widths(dk, dv))
    return lin_padded("linattn_chunk_forward", Lin::gla, q, k, v, g, nullptr, nullptr, nullptr, out, B, H, N, dk, dv,
                      chunk, dtype, segments, workspace, workspace_bytes, stream);
  return lin_forward("linattn_chunk_forward", false, q, k, v, g, nullptr, nullptr, out, B, H, N, dk, dv, chunk,
                     dtype, segments, 0, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int linattn_chunk_forward_state(const void* q, const void* k, const void* v, const float* g, void* out, int64_t B,
                                int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype,
                                int64_t segments, const float* state_in, float* state_out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return lin_forward("linattn_chunk_forward_state", false, q, k, v, g, nullptr, nullptr, out, B, H, N, dk, dv,
                     chunk, dtype, segments, 0, state_in, state_out, workspace, workspace_bytes, stream);
}

int linattn_decode_step(const void* q, const void* k, const void* v, const float* g, void* out, float* state,
                        int64_t B, int64_t H, int64_t dk, int64_t dv, int dtype, void* stream) {
  const char* fn = "linattn_decode_step";
  int st = dec_check(fn, B, H, dk, dv, dtype);
  if (st != LM_OK) return st;
  if (!g) return fail(LM_EINVAL, "%s: null pointer argument", fn);
  if (!aligned(g, 4)) return fail(LM_EINVAL, "%s: misaligned g", fn);
  lm::DecodeLaunch La{};
  La.q = q;
  La.k = k;
  La.v = v;
  La.g = g;
  La.out = out;
  La.state = state;
  La.B = B;
  La.H = H;
  La.D = dk;
  La.bf16 = dtype == LM_BF16;
  return dec_run(fn, false, false, La, dk, (size_t)dk * dv, stream);
}

size_t ccq_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype,
                           int64_t segments) {
  if (!native_widths(dk, dv)) return lin_padded_bytes("ccq_forward", Lin::ccq, B, H, N, dk, dv, chunk, dtype, segments);
  if (lin_check_shape("ccq_forward", B, H, N, dk, dv, chunk, dtype, segments, true) != LM_OK) return 0;
  return lin_layout(B, H, N, dk, true, segments).total;
}

int ccq_forward(const void* q, const void* k, const void* v, const float* g, const float* w_lambda,
                const float* b_lambda, void* out, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                int64_t chunk, int dtype, int64_t segments, void* workspace, size_t workspace_bytes,
                void* stream) {
  if (!native_widths(dk, dv))
    return lin_padded("ccq_forward", Lin::ccq, q, k, v, g, nullptr, w_lambda, b_lambda, out, B, H, N, dk, dv, chunk,
                      dtype, segments, workspace, workspace_bytes, stream);
  return lin_forward("ccq_forward", true, q, k, v, g, w_lambda, b_lambda, out, B, H, N, dk, dv, chunk, dtype,
                     segments, 0, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int ccq_forward_state(const void* q, const void* k, const void* v, const float* g, const float* w_lambda,
                      const float* b_lambda, void* out, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                      int64_t chunk, int dtype, int64_t segments, int64_t t_in, const float* state_in,
                      float* state_out, void* workspace, size_t workspace_bytes, void* stream) {
  return lin_forward("ccq_forward_state", true, q, k, v, g, w_lambda, b_lambda, out, B, H, N, dk, dv, chunk,
                     dtype, segments, t_in, state_in, state_out, workspace, workspace_bytes, stream);
}

int ccq_decode_step(const void* q, const void* k, const void* v, const float* g, const float* w_lambda,
                    const float* b_lambda, void* out, float* state, int64_t B, int64_t H, int64_t dk, int64_t dv,
                    int64_t t_prev, int dtype, void* stream) {
  const char* fn = "ccq_decode_step";
  int st = dec_check(fn, B, H, dk, dv, dtype);
  if (st != LM_OK) return st;
  if (!g || !w_lambda || !b_lambda) return fail(LM_EINVAL, "%s: null pointer argument", fn);
  if (!aligned(g, 4) || !aligned(w_lambda, 4) || !aligned(b_lambda, 4))
    return fail(LM_EINVAL, "%s: misaligned parameter pointer", fn);
  if (t_prev < 0 || t_prev > (int64_t(1) << 40))
    return fail(LM_EINVAL, "%s: t_prev must be in [0, 2^40] (got %lld)", fn, (long long)t_prev);
  lm::DecodeLaunch La{};
  La.q = q;
  La.k = k;
  La.v = v;
  La.g = g;
  La.w_lambda = w_lambda;
  La.b_lambda = b_lambda;
  La.out = out;
  La.state = state;
  La.B = B;
  La.H = H;
  La.D = dk;
  La.t_now = t_prev + 1;
  La.bf16 = dtype == LM_BF16;
  return dec_run(fn, false, true, La, dk, (size_t)dk * dv + (size_t)dk * dk + dk, stream);
}

size_t deltanet_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype,
                                int64_t segments) {
  if (!native_widths(dk, dv))
    return lin_padded_bytes("deltanet_chunk_forward", Lin::delta, B, H, N, dk, dv, chunk, dtype, segments);
  if (delta_check_shape("deltanet_chunk_forward", B, H, N, dk, dv, chunk, dtype, segments) != LM_OK) return 0;
  return delta_layout(B, H, N, dk, dv, dtype, false, segments).total;
}

int deltanet_chunk_forward(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           void* out, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                           int dtype, int64_t segments, void* workspace, size_t workspace_bytes, void* stream) {
  if (!native_widths(dk, dv))
    return lin_padded("deltanet_chunk_forward", Lin::delta, q, k, v, g, beta, nullptr, nullptr, out, B, H, N, dk, dv,
                      chunk, dtype, segments, workspace, workspace_bytes, stream);
  return delta_forward("deltanet_chunk_forward", false, q, k, v, g, beta, nullptr, nullptr, out, B, H, N, dk, dv,
                       chunk, dtype, segments, 0, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int deltanet_forward_state(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           void* out, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                           int dtype, int64_t segments, const float* state_in, float* state_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return delta_forward("deltanet_forward_state", false, q, k, v, g, beta, nullptr, nullptr, out, B, H, N, dk, dv,
                       chunk, dtype, segments, 0, state_in, state_out, workspace, workspace_bytes, stream);
}

size_t ccq_deltanet_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                                    int dtype, int64_t segments) {
  if (!native_widths(dk, dv))
    return lin_padded_bytes("ccq_deltanet_forward", Lin::ccq_delta, B, H, N, dk, dv, chunk, dtype, segments);
  if (delta_check_shape("ccq_deltanet_forward", B, H, N, dk, dv, chunk, dtype, segments) != LM_OK) return 0;
  return delta_layout(B, H, N, dk, dv, dtype, true, segments).total;
}

int ccq_deltanet_forward(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* w_lambda, const float* b_lambda, void* out, int64_t B, int64_t H, int64_t N,
                         int64_t dk, int64_t dv, int64_t chunk, int dtype, int64_t segments, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!native_widths(dk, dv))
    return lin_padded("ccq_deltanet_forward", Lin::ccq_delta, q, k, v, g, beta, w_lambda, b_lambda, out, B, H, N, dk,
                      dv, chunk, dtype, segments, workspace, workspace_bytes, stream);
  return delta_forward("ccq_deltanet_forward", true, q, k, v, g, beta, w_lambda, b_lambda, out, B, H, N, dk, dv,
                       chunk, dtype, segments, 0, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int ccq_deltanet_forward_state(const void* q, const void* k, const void* v, const float* g, const float* beta,
                               const float* w_lambda, const float* b_lambda, void* out, int64_t B, int64_t H,
                               int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype, int64_t segments,
                               int64_t t_in, const float* state_in, float* state_out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return delta_forward("ccq_deltanet_forward_state", true, q, k, v, g, beta, w_lambda, b_lambda, out, B, H, N, dk,
                       dv, chunk, dtype, segments, t_in, state_in, state_out, workspace, workspace_bytes, stream);
}

size_t linattn_vec_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                                   int dtype, int64_t segments) {
  if (!native_widths(dk, dv))
    return lin_padded_bytes("linattn_vec_forward", Lin::vec, B, H, N, dk, dv, chunk, dtype, segments);
  if (lin_check_shape("linattn_vec_forward", B, H, N, dk, dv, chunk, dtype, segments) != LM_OK) return 0;
  return vec_layout(B, H, N, dk, segments).total;
}


int linattn_vec_forward(const void* q, const void* k, const void* v, const float* g, void* out, int64_t B, int64_t H,
                        int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype, int64_t segments,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!native_widths(dk, dv))
    return lin_padded("linattn_vec_forward", Lin::vec, q, k, v, g, nullptr, nullptr, nullptr, out, B, H, N, dk, dv,
                      chunk, dtype, segments, workspace, workspace_bytes, stream);
  return vec_forward("linattn_vec_forward", q, k, v, g, out, B, H, N, dk, dv, chunk, dtype, segments, nullptr,
                     nullptr, workspace, workspace_bytes, stream);
}

int linattn_vec_forward_state(const void* q, const void* k, const void* v, const float* g, void* out, int64_t B,
                              int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype,
                              int64_t segments, const float* state_in, float* state_out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return vec_forward("linattn_vec_forward_state", q, k, v, g, out, B, H, N, dk, dv, chunk, dtype, segments,
                     state_in, state_out, workspace, workspace_bytes, stream);
}

int linattn_vec_decode_step(const void* q, const void* k, const void* v, const float* g, void* out, float* state,
                            int64_t B, int64_t H, int64_t dk, int64_t dv, int dtype, void* stream) {
  const char* fn = "linattn_vec_decode_step";
  int st = dec_check(fn, B, H, dk, dv, dtype);
  if (st != LM_OK) return st;
  if (!g) return fail(LM_EINVAL, "%s: null pointer argument", fn);
  if (!aligned(g, 4)) return fail(LM_EINVAL, "%s: misaligned g", fn);
  lm::DecodeLaunch La{};
  La.q = q;
  La.k = k;
  La.v = v;
  La.g = g;
  La.vector_gates = true;
  La.out = out;
  La.state = state;
  La.B = B;
  La.H = H;
  La.D = dk;
  La.bf16 = dtype == LM_BF16;
  return dec_run(fn, false, false, La, dk, (size_t)dk * dv, stream);
}

// The dedicated bf16 backward kernel: d_k = d_v = 128, rows addressed with
// 32-bit byte offsets within one (b, h) block.
static bool lin_bwd_bf16(int64_t dk, int64_t dv, int64_t N, int dtype) {
  return dtype == LM_BF16 && dk == 128 && dv == 128 && (N + 64) * 128 * 2 < ((int64_t)1 << 31);
}
// It runs one sweep per (b, h) and direction with no segments (2 B H
// workgroups, one per CU), so below about 32 sequences the chunk passes, which
// cut each sequence into segments, are faster; a carried state takes it always.
constexpr int64_t kBwdFusedMinBH = 32;
static bool lin_bwd_fused(int64_t B, int64_t H, int64_t dk, int64_t dv, int64_t N, int dtype, bool stateful) {
  return lin_bwd_bf16(dk, dv, N, dtype) && (stateful || B * H >= kBwdFusedMinBH);
}

size_t linattn_backward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                                        int dtype, int64_t segments) {
  if (lin_check_shape("linattn_chunk_backward", B, H, N, dk, dv, chunk, dtype, segments) != LM_OK) return 0;
  // the dedicated kernel: k . dk per token and the sums over slices of tokens
  // (with fewer sequences the chunk passes' workspace, which also serves a
  // call with a carried state)
  if (lin_bwd_fused(B, H, dk, dv, N, dtype, false))
    return align_up((size_t)B * H * N * 4) + align_up((size_t)B * H * lm::gate_slices(N) * 4);
  // float32 tensors: 5 for the reversed passes, and for bf16 inputs 7 more
  // (float32 copies of q, k, v, do and the gradients before rounding)
  const size_t t = align_up((size_t)B * H * N * dk * 4);
  return (dtype == LM_BF16 ? 12 : 5) * t + align_up((size_t)B * H * N * 4) +
         lin_layout(B, H, N, dk, false, segments).total;
}

static int lin_backward(const char* fn, const void* q, const void* k, const void* v, const float* g, const void* dout,
                        const float* state_in, const float* dstate_out, void* dq, void* dk, void* dv, float* dg,
                        float* dstate_in, int64_t B, int64_t H, int64_t N, int64_t dkk, int64_t dvv, int64_t chunk,
                        int dtype, int64_t segments, void* workspace, size_t workspace_bytes, void* stream) {
  int st = lin_check_shape(fn, B, H, N, dkk, dvv, chunk, dtype, segments);
  if (st != LM_OK) return st;
  if (!q || !k || !v || !g || !dout || !dq || !dk || !dv || !dg || !workspace)
    return fail(LM_EINVAL, "%s: null pointer argument", fn);
  const bool stateful = state_in || dstate_out || dstate_in;
  if (stateful && !lin_bwd_bf16(dkk, dvv, N, dtype))
    return fail(LM_EUNSUPPORTED, "%s: a carried state is implemented for bf16 with dk = dv = 128", fn);
  const size_t ns = (size_t)B * H * dkk * dvv * 4;
  for (const float* p : {state_in, dstate_out, static_cast<const float*>(dstate_in)})
    if (p && !aligned(p, 16)) return fail(LM_EINVAL, "%s: misaligned state pointer (16 bytes needed)", fn);
  const void* ptrs16[] = {q, k, v, dout, dq, dk, dv, workspace};
  for (const void* p : ptrs16)
    if (!aligned(p, 16)) return fail(LM_EINVAL, "%s: misaligned pointer (tensors need 16 bytes)", fn);
  if (!aligned(g, 4) || !aligned(dg, 4)) return fail(LM_EINVAL, "%s: misaligned g or dg", fn);
  const size_t es = esize(dtype), nt = (size_t)B * H * N * dkk * es, ng = (size_t)B * H * N * 4;
  const size_t t = align_up((size_t)B * H * N * dkk * 4);
  const size_t need = linattn_backward_workspace_bytes(B, H, N, dkk, dvv, chunk, dtype, segments);
  if (workspace_bytes < need)
    return fail(LM_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
  // outputs must not overlap each other, the inputs or the workspace
  const void* outs[] = {dq, dk, dv, dg};
  const size_t nout[] = {nt, nt, nt, ng};
  const void* ins[] = {q, k, v, dout, g, workspace};
  const size_t nin[] = {nt, nt, nt, nt, ng, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], nout[i], ins[j], nin[j]))
        return fail(LM_EINVAL, "%s: an output overlaps an input or the workspace", fn);
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], nout[i], outs[j], nout[j])) return fail(LM_EINVAL, "%s: outputs overlap", fn);
  }
  // the states: inputs state_in, dstate_out; output dstate_in
  for (const float* p : {state_in, dstate_out}) {
    if (!p) continue;
    for (int i = 0; i < 4; ++i)
      if (overlap(outs[i], nout[i], p, ns)) return fail(LM_EINVAL, "%s: an output overlaps a state input", fn);
    if (dstate_in && overlap(dstate_in, ns, p, ns))
      return fail(LM_EINVAL, "%s: dstate_in overlaps a state input", fn);
  }
  if (dstate_in) {
    for (int i = 0; i < 4; ++i)
      if (overlap(outs[i], nout[i], dstate_in, ns)) return fail(LM_EINVAL, "%s: outputs overlap", fn);
    for (int j = 0; j < 6; ++j)
      if (overlap(dstate_in, ns, ins[j], nin[j]))
        return fail(LM_EINVAL, "%s: dstate_in overlaps an input or the workspace", fn);
  }
  if (lin_bwd_fused(B, H, dkk, dvv, N, dtype, stateful)) {
    lm::BwdBf16Launch Lb;
    Lb.q = q;
    Lb.k = k;
    Lb.v = v;
    Lb.g = g;
    Lb.dout = dout;
    Lb.dq = dq;
    Lb.dk = dk;
    Lb.dv = dv;
    Lb.dg = dg;
    Lb.xk = static_cast<float*>(workspace);
    Lb.tot = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up((size_t)B * H * N * 4));
    Lb.state_in = state_in;
    Lb.dstate_out = dstate_out;
    Lb.dstate_in = dstate_in;
    Lb.B = B;
    Lb.H = H;
    Lb.N = N;
    hipError_t e = lm::linattn_backward_bf16_launch(Lb, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(LM_EHIP, "%s: %s", fn, hipGetErrorString(e));
    return ok();
  }
  char* ws = static_cast<char*>(workspace);
  const LinLayout LL = lin_layout(B, H, N, dkk, false, segments);
  lm::BwdLaunch La;
  const int nten = dtype == LM_BF16 ? 12 : 5;
  La.fwd.agg = reinterpret_cast<float*>(ws + nten * t + align_up(ng) + LL.agg);
  La.fwd.w_lambda = nullptr;
  La.fwd.b_lambda = nullptr;
  La.fwd.B = B;
  La.fwd.H = H;
  La.fwd.N = N;
  La.fwd.D = dkk;
  La.fwd.P = LL.plan.P;
  La.fwd.seg_len = LL.plan.seg_len;
  La.fwd.R = LL.R;
  La.fwd.bf16 = dtype == LM_BF16;
  La.q = q;
  La.k = k;
  La.v = v;
  La.g = g;
  La.dout = dout;
  La.dq = dq;
  La.dk = dk;
  La.dv = dv;
  La.dg = dg;
  float* f[12];
  for (int i = 0; i < nten; ++i) f[i] = reinterpret_cast<float*>(ws + i * t);
  for (int i = nten; i < 12; ++i) f[i] = nullptr;
  La.rq = f[0];
  La.rk = f[1];
  La.rv = f[2];
  La.rdo = f[3];
  La.rout = f[4];
  La.uq = f[5];
  La.uk = f[6];
  La.uv = f[7];
  La.udo = f[8];
  La.udq = f[9];
  La.udk = f[10];
  La.udv = f[11];
  La.rg = reinterpret_cast<float*>(ws + nten * t);
  La.B = B;
  La.H = H;
  La.N = N;
  La.D = dkk;
  La.bf16 = dtype == LM_BF16;
  hipError_t e = lm::linattn_backward_launch(La, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LM_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

int linattn_chunk_backward(const void* q, const void* k, const void* v, const float* g, const void* dout, void* dq,
                           void* dk, void* dv, float* dg, int64_t B, int64_t H, int64_t N, int64_t dkk, int64_t dvv,
                           int64_t chunk, int dtype, int64_t segments, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return lin_backward("linattn_chunk_backward", q, k, v, g, dout, nullptr, nullptr, dq, dk, dv, dg, nullptr, B, H, N,
                      dkk, dvv, chunk, dtype, segments, workspace, workspace_bytes, stream);
}

int linattn_chunk_backward_state(const void* q, const void* k, const void* v, const float* g, const void* dout,
                                 const float* state_in, const float* dstate_out, void* dq, void* dk, void* dv,
                                 float* dg, float* dstate_in, int64_t B, int64_t H, int64_t N, int64_t dkk,
                                 int64_t dvv, int64_t chunk, int dtype, int64_t segments, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return lin_backward("linattn_chunk_backward_state", q, k, v, g, dout, state_in, dstate_out, dq, dk, dv, dg,
                      dstate_in, B, H, N, dkk, dvv, chunk, dtype, segments, workspace, workspace_bytes, stream);
}

size_t gma_backward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv, int causal,
                                    int dtype) {
  if (gma_bwd_check("gma_backward", B, H, N, d, K, dv, causal, 0.f, dtype) != LM_OK) return 0;
  return gma_bwd_layout(B, H, N, d, K, dv, causal).total;
}

int gma_backward(const void* q, const void* k, const void* v, const float* mu, const float* log_var,
                 const float* logit_pi, const void* dout, void* dq, void* dk, void* dv, float* dmu, float* dlog_var,
                 float* dlogit_pi, int64_t B, int64_t H, int64_t N, int64_t d, int64_t K, int64_t dvv, int causal,
                 float eps, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "gma_backward";
  int st = gma_bwd_check(fn, B, H, N, d, K, dvv, causal, eps, dtype);
  if (st != LM_OK) return st;
  if (!q || !k || !v || !mu || !log_var || !logit_pi || !dout || !dq || !dk || !dv || !dmu || !dlog_var ||
      !dlogit_pi || !workspace)
    return fail(LM_EINVAL, "%s: null pointer argument", fn);
  const void* p16[] = {q, k, v, dout, dq, dk, dv, workspace};
  for (const void* p : p16)
    if (!aligned(p, 16)) return fail(LM_EINVAL, "%s: misaligned pointer (tensors need 16 bytes)", fn);
  const void* p4[] = {mu, log_var, logit_pi, dmu, dlog_var, dlogit_pi};
  for (const void* p : p4)
    if (!aligned(p, 4)) return fail(LM_EINVAL, "%s: misaligned parameter pointer", fn);
  const GmaBwdLayout L = gma_bwd_layout(B, H, N, d, K, dvv, causal);
  if (workspace_bytes < L.total)
    return fail(LM_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, L.total);
  // outputs must not overlap each other, the inputs or the workspace
  const size_t nt = (size_t)B * H * N * d * esize(dtype), np = (size_t)H * K * d * 4, nl = (size_t)H * K * 4;
  const void* outs[] = {dq, dk, dv, dmu, dlog_var, dlogit_pi};
  const size_t nout[] = {nt, nt, nt, np, np, nl};
  const void* ins[] = {q, k, v, dout, mu, log_var, logit_pi, workspace};
  const size_t nin[] = {nt, nt, nt, nt, np, np, nl, L.total};
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlap(outs[i], nout[i], ins[j], nin[j]))
        return fail(LM_EINVAL, "%s: an output overlaps an input or the workspace", fn);
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], nout[i], outs[j], nout[j])) return fail(LM_EINVAL, "%s: outputs overlap", fn);
  }
  char* ws = static_cast<char*>(workspace);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  lm::GmaBwdLaunch La{};
  lm::BwdLaunch& Bw = La.bwd;
  Bw.fwd.agg = F(L.agg);
  Bw.fwd.w_lambda = nullptr;
  Bw.fwd.b_lambda = nullptr;
  Bw.fwd.B = B;
  Bw.fwd.H = H;
  Bw.fwd.N = L.NN;
  Bw.fwd.D = L.DL;
  Bw.fwd.P = L.lin.plan.P;
  Bw.fwd.seg_len = L.lin.plan.seg_len;
  Bw.fwd.R = L.lin.R;
  Bw.fwd.bf16 = false;
  Bw.fwd.ccq = false;
  Bw.rq = F(L.inner[0]);
  Bw.rk = F(L.inner[1]);
  Bw.rv = F(L.inner[2]);
  Bw.rdo = F(L.inner[3]);
  Bw.rout = F(L.inner[4]);
  Bw.rg = F(L.rg);
  Bw.dg = nullptr;
  Bw.B = B;
  Bw.H = H;
  Bw.N = L.NN;
  Bw.D = L.DL;
  Bw.bf16 = false;
  La.q = q;
  La.k = k;
  La.v = v;
  La.dout = dout;
  La.mu = mu;
  La.log_var = log_var;
  La.logit_pi = logit_pi;
  La.dq = dq;
  La.dk = dk;
  La.dv = dv;
  La.dmu = dmu;
  La.dlog_var = dlog_var;
  La.dlogit_pi = dlogit_pi;
  La.iv = F(L.iv);
  La.cst = F(L.cst);
  La.gq = F(L.rows[0]);
  La.gk = F(L.rows[1]);
  La.vx = F(L.rows[2]);
  La.y = F(L.rows[3]);
  La.dy = F(L.rows[4]);
  La.dgq = F(L.rows[5]);
  La.dgk = F(L.rows[6]);
  La.dvx = F(L.rows[7]);
  La.ones = F(L.ones);
  La.part = F(L.part);
  La.sums = F(L.sums);
  La.B = B;
  La.H = H;
  La.N = N;
  La.D = d;
  La.K = K;
  La.DL = L.DL;
  La.nseg = L.nseg;
  La.seg_len = L.seg_len;
  La.NN = L.NN;
  La.NF = L.NF;
  La.NVB = L.NVB;
  La.bstride = (size_t)B * H * L.NN * 128;
  if (L.wide) {
    La.tq = F(L.tmp[0]);
    La.tk = F(L.tmp[1]);
    La.tv = F(L.tmp[2]);
  }
  La.causal = causal;
  La.eps = eps;
  La.bf16 = dtype == LM_BF16;
  hipError_t e = lm::gma_backward_launch(La, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LM_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

size_t ccq_backward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                                    int dtype) {
  if (lin_check_shape("ccq_backward", B, H, N, dk, dv, chunk, dtype, 0) != LM_OK) return 0;
  return ccq_bwd_layout(B, H, N, dk, dtype).total;
}

int ccq_backward(const void* q, const void* k, const void* v, const float* g, const float* w_lambda,
                 const float* b_lambda, const void* dout, void* dq, void* dk, void* dv, float* dg, float* dw_lambda,
                 float* db_lambda, int64_t B, int64_t H, int64_t N, int64_t dkk, int64_t dvv, int64_t chunk,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "ccq_backward";
  int st = lin_check_shape(fn, B, H, N, dkk, dvv, chunk, dtype, 0);
  if (st != LM_OK) return st;
  if (!q || !k || !v || !g || !w_lambda || !b_lambda || !dout || !dq || !dk || !dv || !dg || !dw_lambda ||
      !db_lambda || !workspace)
    return fail(LM_EINVAL, "%s: null pointer argument", fn);
  const void* p16[] = {q, k, v, dout, dq, dk, dv, workspace};
  for (const void* p : p16)
    if (!aligned(p, 16)) return fail(LM_EINVAL, "%s: misaligned pointer (tensors need 16 bytes)", fn);
  const void* p4[] = {g, w_lambda, b_lambda, dg, dw_lambda, db_lambda};
  for (const void* p : p4)
    if (!aligned(p, 4)) return fail(LM_EINVAL, "%s: misaligned float pointer", fn);
  const CcqBwdLayout L = ccq_bwd_layout(B, H, N, dkk, dtype);
  if (workspace_bytes < L.total)
    return fail(LM_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, L.total);
  const size_t nt = (size_t)B * H * N * dkk * esize(dtype), ng = (size_t)B * H * N * 4,
               nw = (size_t)H * dkk * 4, nb = (size_t)H * 4;
  const void* outs[] = {dq, dk, dv, dg, dw_lambda, db_lambda};
  const size_t nout[] = {nt, nt, nt, ng, nw, nb};
  const void* ins[] = {q, k, v, dout, g, w_lambda, b_lambda, workspace};
  const size_t nin[] = {nt, nt, nt, nt, ng, nw, nb, L.total};
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlap(outs[i], nout[i], ins[j], nin[j]))
        return fail(LM_EINVAL, "%s: an output overlaps an input or the workspace", fn);
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], nout[i], outs[j], nout[j])) return fail(LM_EINVAL, "%s: outputs overlap", fn);
  }
  char* ws = static_cast<char*>(workspace);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  lm::CcqBwdLaunch La{};
  lm::BwdLaunch& Bw = La.bwd;
  Bw.fwd.agg = F(L.agg);
  Bw.fwd.w_lambda = nullptr;
  Bw.fwd.b_lambda = nullptr;
  Bw.fwd.B = B;
  Bw.fwd.H = H;
  Bw.fwd.N = N;
  Bw.fwd.D = dkk;
  Bw.fwd.P = L.lin.plan.P;
  Bw.fwd.seg_len = L.lin.plan.seg_len;
  Bw.fwd.R = L.lin.R;
  Bw.fwd.bf16 = false;
  Bw.fwd.ccq = false;
  Bw.g = g;
  Bw.dg = dg;
  Bw.B = B;
  Bw.H = H;
  Bw.N = N;
  Bw.D = dkk;
  Bw.bf16 = false;
  int r = 0;
  float** rowp[] = {&La.m, &La.mq, &La.s, &La.qc, &La.u, &La.dkg, &La.mu, &La.vr1, &La.vr2, &La.dm, &La.sdm, &La.r1,
                    &La.r2, &Bw.rq, &Bw.rk, &Bw.rv, &Bw.rdo, &Bw.rout};
  for (float** p : rowp) *p = F(L.rows[r++]);
  if (dtype == LM_BF16) {
    La.fk = F(L.rows[r++]);
    La.fv = F(L.rows[r++]);
    La.fdo = F(L.rows[r++]);
    La.dvg = F(L.rows[r++]);
  }
  La.lam = F(L.cols[0]);
  La.ones = F(L.cols[1]);
  Bw.rg = F(L.cols[2]);
  La.csum = F(L.csum);
  La.part = F(L.part);
  La.q = q;
  La.k = k;
  La.v = v;
  La.dout = dout;
  La.w = w_lambda;
  La.b = b_lambda;
  La.dq = dq;
  La.dk = dk;
  La.dv = dv;
  La.dw = dw_lambda;
  La.db = db_lambda;
  La.B = B;
  La.H = H;
  La.N = N;
  La.D = dkk;
  La.nch = L.nch;
  La.clen = L.clen;
  La.nblk = L.nblk;
  La.blen = L.blen;
  La.fused = lin_bwd_fused(B, H, dkk, dvv, N, dtype, false);
  La.bf16 = dtype == LM_BF16;
  hipError_t e = lm::ccq_backward_launch(La, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LM_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // extern "C"
