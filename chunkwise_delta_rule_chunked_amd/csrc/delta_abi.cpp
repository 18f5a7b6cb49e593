// C ABI of the delta-rule library: argument validation, workspace layout and kernel
// dispatch.  Every entry point validates everything before enqueuing any work and
// never allocates device memory.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/delta.h"
#include "kernels.h"

using delta::BwdParams;
using delta::DecodeParams;
using delta::FwdParams;
using delta::LayerParams;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, unsigned a) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

size_t esize(int dtype) { return dtype == DELTA_BF16 ? 2 : 4; }

// Shape checks common to all entry points.
int check_shape(const delta_shape* s) {
  if (!s) return DELTA_ERR_NULL_ARG;
  if (s->B < 0 || s->L < 0 || s->H < 0 || s->n_h < 1) return DELTA_ERR_BAD_SHAPE;
  if (s->dtype != DELTA_F32 && s->dtype != DELTA_BF16) return DELTA_ERR_UNSUPPORTED_DIM;
  if (s->dk != 16 && s->dk != 32 && s->dk != 64 && s->dk != 128) return DELTA_ERR_UNSUPPORTED_DIM;
  if (s->dv < 16 || s->dv > 256 || s->dv % 16 != 0) return DELTA_ERR_UNSUPPORTED_DIM;
  // grid sizes and 64-bit element counts stay well inside what the kernels index
  const long long Lx = (long long)s->L * s->n_h;
  if (Lx > (1LL << 31) || (long long)s->B * s->H > (1LL << 24)) return DELTA_ERR_BAD_SHAPE;
  return DELTA_OK;
}

int check_chunk(const delta_shape* s) {
  if (s->chunk != 16 && s->chunk != 32 && s->chunk != 48 && s->chunk != 64) return DELTA_ERR_UNSUPPORTED_DIM;
  if (s->chunk % s->n_h != 0) return DELTA_ERR_BAD_SHAPE;
  const long long NT = ((long long)s->L * s->n_h + s->chunk - 1) / s->chunk;
  if ((long long)s->B * s->H * NT > (1LL << 31) - 1) return DELTA_ERR_BAD_SHAPE;
  // the kernels address one chunk of one sequence with 32-bit element offsets
  if ((long long)s->chunk * s->H * (s->dk > s->dv ? s->dk : s->dv) >= (1LL << 31)) return DELTA_ERR_BAD_SHAPE;
  return DELTA_OK;
}

FwdParams make_params(const delta_shape* s) {
  FwdParams p;
  memset(&p, 0, sizeof(p));
  p.B = s->B;
  p.L = s->L;
  p.H = s->H;
  p.DK = s->dk;
  p.DV = s->dv;
  p.nh = s->n_h;
  p.C = s->chunk;
  p.Lx = s->L * s->n_h;
  p.NT = (p.Lx + p.C - 1) / p.C;
  p.scale = s->scale;
  // Sequence split of the inter-chunk pass: enough segments per head that the output launch
  // has about 256 workgroups (one per compute unit), each segment at least one chunk.  A
  // function of the shape alone, so results do not depend on the device.
  const long long units = (long long)p.B * p.H * ((p.DV / 16 + (p.DV <= 64 ? 4 : 8) - 1) / (p.DV <= 64 ? 4 : 8));
  long long P = units > 0 && p.NT > 1 ? 256 / units : 1;
  if (P < 1) P = 1;
  if (P > p.NT) P = p.NT > 0 ? p.NT : 1;
  p.NS = p.NT > 0 ? (int)((p.NT + P - 1) / P) : 1;
  p.P = p.NT > 0 ? (p.NT + p.NS - 1) / p.NS : 1;
  return p;
}

size_t t_bytes(const FwdParams& p, size_t es) { return (size_t)p.B * p.H * p.NT * p.C * p.C * es; }
size_t gc_bytes(const FwdParams& p) { return (size_t)p.B * p.H * p.NT * p.C * 4; }
// segment summaries and start states (only with a sequence split)
size_t sm_bytes(const FwdParams& p) { return p.P > 1 ? (size_t)p.B * p.H * p.P * p.DK * (p.DV + p.DK) * 4 : 0; }
size_t sst_bytes(const FwdParams& p) { return p.P > 1 ? (size_t)p.B * p.H * p.P * p.DK * p.DV * 4 : 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? DELTA_OK : DELTA_ERR_HIP; }

// Opt-in switches, read from the environment at every call:
//   DELTA_VALIDATE=1    check beta and the log gates before enqueuing work (validate.hip); a
//                       value outside the contract returns DELTA_ERR_BAD_VALUE with nothing
//                       written.  The check waits for the stream, so the call is synchronous.
//   DELTA_FAULT=launch  every entry point that has work to enqueue fails as if its first launch
//                       had failed: DELTA_ERR_HIP, nothing enqueued (for testing error paths).
bool env_is(const char* name, const char* value) {
  const char* e = getenv(name);
  return e && strcmp(e, value) == 0;
}
bool validate_on() { return env_is("DELTA_VALIDATE", "1"); }
int launch_guard() { return env_is("DELTA_FAULT", "launch") ? DELTA_ERR_HIP : DELTA_OK; }

// The validation pass on the device: the flag words go to `flags` (VALIDATE_BLOCKS words of the
// caller's workspace, overwritten afterwards by the pass itself), then are read back.
int validate_device(const float* beta, size_t nbeta, const float* glog, size_t ngate, void* flags, hipStream_t st) {
  if (nbeta + ngate == 0) return DELTA_OK;
  unsigned* f = static_cast<unsigned*>(flags);
  if (delta::launch_validate(beta, (long)nbeta, glog, (long)ngate, f, st) != hipSuccess) return DELTA_ERR_HIP;
  unsigned h[delta::VALIDATE_BLOCKS];
  if (hipMemcpyAsync(h, f, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess) return DELTA_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return DELTA_ERR_HIP;
  for (unsigned x : h)
    if (x) return DELTA_ERR_BAD_VALUE;
  return DELTA_OK;
}

// The same check for the decode steps, which take no workspace: their beta and gate arrays are
// one value per (sequence, head) or per key channel, read back and checked on the host.
int validate_small(const float* beta, size_t nbeta, const float* glog, size_t ngate, hipStream_t st) {
  std::vector<float> hb(nbeta), hg(ngate);
  if (nbeta && hipMemcpyAsync(hb.data(), beta, nbeta * 4, hipMemcpyDeviceToHost, st) != hipSuccess) return DELTA_ERR_HIP;
  if (ngate && hipMemcpyAsync(hg.data(), glog, ngate * 4, hipMemcpyDeviceToHost, st) != hipSuccess) return DELTA_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return DELTA_ERR_HIP;
  for (float x : hb)
    if (!__builtin_isfinite(x)) return DELTA_ERR_BAD_VALUE;
  for (float x : hg)
    if (x != x || x == __builtin_inff()) return DELTA_ERR_BAD_VALUE;
  return DELTA_OK;
}

}  // namespace

extern "C" {

int delta_fwd_workspace_bytes(const delta_shape* s, size_t* bytes) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_chunk(s))) return rc;
  if (!bytes) return DELTA_ERR_NULL_ARG;
  const FwdParams p = make_params(s);
  // T (element type of the inputs), the gate prefix, then the segment summaries and segment
  // start states of the inter-chunk pass
  *bytes = align_up(t_bytes(p, esize(s->dtype))) + align_up(gc_bytes(p)) + align_up(sm_bytes(p)) +
           align_up(sst_bytes(p));
  return DELTA_OK;
}

}  // extern "C"

namespace {

// Phases a forward call may cover; each names the tensors it reads or writes.
enum Phase {
  PH_ALL = 0,      // the whole pass: q, k, v, beta, g_log, S0, O, S_final
  PH_INTRA = 1,    // k, beta, g_log
  PH_INTER = 2,    // q, k, v, S0, O, S_final
  PH_SUMMARY = 3,  // k, v, S0
  PH_COMBINE = 4,  // workspace only
  PH_OUTPUTS = 5   // q, k, v, S0, O, S_final
};

// Validates a forward call and fills p.  Pointers the phase does not use are ignored.
int prepare_fwd(const delta_shape* s, int phase, const void* q, const void* k, const void* v,
                const float* beta, const float* g_log, const float* S0, void* O, float* S_final,
                void* workspace, size_t workspace_bytes, FwdParams& p) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_chunk(s))) return rc;
  p = make_params(s);
  const bool use_intra = phase == PH_ALL || phase == PH_INTRA;
  const bool use_q = phase == PH_ALL || phase == PH_INTER || phase == PH_OUTPUTS, use_k = phase != PH_COMBINE;
  const bool use_vs = phase == PH_ALL || phase == PH_INTER || phase == PH_SUMMARY || phase == PH_OUTPUTS;
  const bool use_out = phase == PH_ALL || phase == PH_INTER || phase == PH_OUTPUTS;
  if (!use_intra) beta = nullptr, g_log = nullptr;
  if (!use_q) q = nullptr;
  if (!use_k) k = nullptr;
  if (!use_vs) v = nullptr, S0 = nullptr;
  if (!use_out) O = nullptr, S_final = nullptr;
  const size_t es = esize(s->dtype);
  const size_t sz_q = (size_t)p.B * p.L * p.H * p.DK * es, sz_k = (size_t)p.B * p.Lx * p.H * p.DK * es,
               sz_v = (size_t)p.B * p.Lx * p.H * p.DV * es, sz_b = (size_t)p.B * p.Lx * p.H * 4,
               sz_g = (size_t)p.B * p.L * p.H * 4, sz_S = (size_t)p.B * p.H * p.DK * p.DV * 4,
               sz_o = (size_t)p.B * p.L * p.H * p.DV * es;
  // a pointer is required when its tensor is not empty
  if ((use_k && sz_k && !k) || (use_q && sz_q && !q) || (use_vs && sz_v && !v) || (use_out && sz_o && !O) ||
      (use_intra && sz_b && !beta))
    return DELTA_ERR_NULL_ARG;
  size_t need = 0;
  delta_fwd_workspace_bytes(s, &need);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DELTA_ERR_WORKSPACE;
  // q, k, v, O, the states and the workspace are moved with 16-byte vector accesses; beta and
  // g_log are read as scalars
  const void* ptrs[] = {q, k, v, S0, O, S_final, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DELTA_ERR_MISALIGNED;
  if (!aligned(beta, 4) || !aligned(g_log, 4)) return DELTA_ERR_MISALIGNED;

  const Range in[] = {range(q, q ? sz_q : 0), range(k, k ? sz_k : 0), range(v, v ? sz_v : 0),
                      range(beta, beta ? sz_b : 0), range(g_log, g_log ? sz_g : 0), range(S0, S0 ? sz_S : 0)};
  const Range ro = range(O, O ? sz_o : 0), rs = range(S_final, S_final ? sz_S : 0), rw = range(workspace, need);
  for (const Range& r : in) {
    if (overlap(ro, r) || overlap(rw, r)) return DELTA_ERR_ALIAS;
    // S_final may be exactly S0 (in-place); any other overlap with an input is an error
    if (overlap(rs, r) && !(S0 && S_final == S0 && r.lo == reinterpret_cast<uintptr_t>(S0))) return DELTA_ERR_ALIAS;
  }
  if (overlap(ro, rs) || overlap(ro, rw) || overlap(rs, rw)) return DELTA_ERR_ALIAS;

  p.q = q;
  p.k = k;
  p.v = v;
  p.beta = beta;
  p.g_log = g_log;
  p.S0 = S0;
  p.O = O;
  p.S_final = S_final;
  p.T = workspace;
  char* ws = static_cast<char*>(workspace);
  size_t off = align_up(t_bytes(p, es));
  p.gc = reinterpret_cast<float*>(ws + off);
  off += align_up(gc_bytes(p));
  p.SM = p.P > 1 ? reinterpret_cast<float*>(ws + off) : nullptr;
  off += align_up(sm_bytes(p));
  p.Sst = p.P > 1 ? reinterpret_cast<float*>(ws + off) : nullptr;
  return DELTA_OK;
}

int run_intra(const FwdParams& p, bool bf, hipStream_t st) {
  if (p.B * p.H * p.NT == 0) return DELTA_OK;
  int rc = launch_guard();
  if (rc) return rc;
  if (validate_on() &&
      (rc = validate_device(p.beta, (size_t)p.B * p.Lx * p.H, p.g_log, p.g_log ? (size_t)p.B * p.L * p.H : 0, p.T, st)))
    return rc;
  return hip_status(delta::launch_intra_chunk(p, bf, false, st));
}

int run_scan(const FwdParams& p, bool bf, int phase, hipStream_t st) {
  if (p.B * p.H == 0) return DELTA_OK;
  // L == 0: no chunks; the output launch still writes S_final = S0 (or zeros)
  if (p.NT == 0 && (phase != delta::SCAN_OUTPUTS || !p.S_final)) return DELTA_OK;
  int rc = launch_guard();
  if (rc) return rc;
  return hip_status(delta::launch_scan_phase(p, bf, phase, st));
}

int run_inter(const FwdParams& p, bool bf, hipStream_t st) {
  int rc;
  if ((rc = run_scan(p, bf, delta::SCAN_SUMMARY, st))) return rc;
  if ((rc = run_scan(p, bf, delta::SCAN_COMBINE, st))) return rc;
  return run_scan(p, bf, delta::SCAN_OUTPUTS, st);
}

}  // namespace

extern "C" {

int delta_fwd(const delta_shape* s, const void* q, const void* k, const void* v, const float* beta,
              const float* g_log, const float* S0, void* O, float* S_final, void* workspace,
              size_t workspace_bytes, void* stream) {
  FwdParams p;
  int rc = prepare_fwd(s, PH_ALL, q, k, v, beta, g_log, S0, O, S_final, workspace, workspace_bytes, p);
  if (rc) return rc;
  const bool bf = s->dtype == DELTA_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = run_intra(p, bf, st))) return rc;
  return run_inter(p, bf, st);
}

int delta_fwd_intra(const delta_shape* s, const void* k, const float* beta, const float* g_log,
                    void* workspace, size_t workspace_bytes, void* stream) {
  FwdParams p;
  int rc = prepare_fwd(s, PH_INTRA, nullptr, k, nullptr, beta, g_log, nullptr, nullptr, nullptr, workspace,
                       workspace_bytes, p);
  if (rc) return rc;
  return run_intra(p, s->dtype == DELTA_BF16, static_cast<hipStream_t>(stream));
}

int delta_fwd_inter(const delta_shape* s, const void* q, const void* k, const void* v, const float* S0,
                    void* O, float* S_final, void* workspace, size_t workspace_bytes, void* stream) {
  FwdParams p;
  int rc = prepare_fwd(s, PH_INTER, q, k, v, nullptr, nullptr, S0, O, S_final, workspace, workspace_bytes, p);
  if (rc) return rc;
  return run_inter(p, s->dtype == DELTA_BF16, static_cast<hipStream_t>(stream));
}

int delta_fwd_segments(const delta_shape* s, int32_t* segments, int32_t* chunks_per_segment) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_chunk(s))) return rc;
  if (!segments || !chunks_per_segment) return DELTA_ERR_NULL_ARG;
  const FwdParams p = make_params(s);
  *segments = p.P;
  *chunks_per_segment = p.NS;
  return DELTA_OK;
}

int delta_fwd_scan_summary(const delta_shape* s, const void* k, const void* v, const float* S0,
                           void* workspace, size_t workspace_bytes, void* stream) {
  FwdParams p;
  int rc = prepare_fwd(s, PH_SUMMARY, nullptr, k, v, nullptr, nullptr, S0, nullptr, nullptr, workspace,
                       workspace_bytes, p);
  if (rc) return rc;
  return run_scan(p, s->dtype == DELTA_BF16, delta::SCAN_SUMMARY, static_cast<hipStream_t>(stream));
}

int delta_fwd_scan_combine(const delta_shape* s, void* workspace, size_t workspace_bytes, void* stream) {
  FwdParams p;
  int rc = prepare_fwd(s, PH_COMBINE, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                       workspace, workspace_bytes, p);
  if (rc) return rc;
  return run_scan(p, s->dtype == DELTA_BF16, delta::SCAN_COMBINE, static_cast<hipStream_t>(stream));
}

int delta_fwd_scan_outputs(const delta_shape* s, const void* q, const void* k, const void* v,
                           const float* S0, void* O, float* S_final, void* workspace,
                           size_t workspace_bytes, void* stream) {
  FwdParams p;
  int rc = prepare_fwd(s, PH_OUTPUTS, q, k, v, nullptr, nullptr, S0, O, S_final, workspace, workspace_bytes,
                       p);
  if (rc) return rc;
  return run_scan(p, s->dtype == DELTA_BF16, delta::SCAN_OUTPUTS, static_cast<hipStream_t>(stream));
}

int delta_chunk_wy(const delta_shape* s, const void* k, const void* v, const float* beta,
                   const float* g_log, float* T, float* W, float* U, float* gc, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_chunk(s))) return rc;
  FwdParams p = make_params(s);
  const size_t es = esize(s->dtype);
  if (p.B * p.H * p.NT > 0 && (!k || !beta || !T || !gc || (U && !v))) return DELTA_ERR_NULL_ARG;
  const void* ptrs[] = {k, v, T, W, U, gc};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DELTA_ERR_MISALIGNED;
  if (!aligned(beta, 4) || !aligned(g_log, 4)) return DELTA_ERR_MISALIGNED;
  const Range in[] = {range(k, (size_t)p.B * p.Lx * p.H * p.DK * es),
                      range(v, v ? (size_t)p.B * p.Lx * p.H * p.DV * es : 0),
                      range(beta, (size_t)p.B * p.Lx * p.H * 4),
                      range(g_log, g_log ? (size_t)p.B * p.L * p.H * 4 : 0)};
  const Range out[] = {range(T, t_bytes(p, 4)), range(gc, gc_bytes(p)),
                       range(W, W ? (size_t)p.B * p.H * p.NT * p.C * p.DK * 4 : 0),
                       range(U, U ? (size_t)p.B * p.H * p.NT * p.C * p.DV * 4 : 0)};
  for (int i = 0; i < 4; ++i) {
    for (const Range& r : in)
      if (overlap(out[i], r)) return DELTA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(out[i], out[j])) return DELTA_ERR_ALIAS;
  }
  p.k = k;
  p.v = v;
  p.beta = beta;
  p.g_log = g_log;
  p.T = T;
  p.gc = gc;
  p.W = W;
  p.U = U;
  const bool bf = s->dtype == DELTA_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.B * p.H * p.NT == 0) return DELTA_OK;
  if ((rc = launch_guard())) return rc;
  if ((rc = hip_status(delta::launch_intra_chunk(p, bf, true, st)))) return rc;
  if (W || U) return hip_status(delta::launch_wy_factors(p, bf, st));
  return DELTA_OK;
}

namespace {
// Workspace of the backward pass.  Where the state scans apply (bf16, d_k = d_v = 128, chunk 64):
// T (bf16), the gate prefix, N = (I + A)^-1 (float32), the segment summaries of the two scans
// (the reverse scan's transition maps are the forward's, transposed) and their start states,
// and per chunk the start state (bf16) and the end-of-chunk state gradient (bf16 and its bf16
// rounding residual).  Otherwise:
// T (float32), the gate prefix, Q K^T * Gam (float32, C x C per chunk) and the two per-chunk
// state arrays in float32.
size_t states_bytes(const FwdParams& p) { return (size_t)p.B * p.H * p.NT * p.DK * p.DV * 4; }
bool bwd_scans(const FwdParams& p, bool bf) { return p.NT > 0 && delta::bwd_scans_apply(p, bf); }
size_t bwd_workspace(const FwdParams& p, bool bf) {
  if (bwd_scans(p, bf))
    return align_up(t_bytes(p, 2)) + align_up(gc_bytes(p)) + align_up(t_bytes(p, 4)) + 2 * align_up(sm_bytes(p)) +
           align_up(sst_bytes(p)) + 3 * align_up(states_bytes(p) / 2);
  return 2 * align_up(t_bytes(p, 4)) + align_up(gc_bytes(p)) + 2 * align_up(states_bytes(p));
}
}  // namespace

int delta_bwd_workspace_bytes(const delta_shape* s, size_t* bytes) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_chunk(s))) return rc;
  if (!bytes) return DELTA_ERR_NULL_ARG;
  *bytes = bwd_workspace(make_params(s), s->dtype == DELTA_BF16);
  return DELTA_OK;
}

int delta_bwd(const delta_shape* s, const void* q, const void* k, const void* v, const float* beta,
              const float* g_log, const float* S0, const void* dO, const float* dS_final, float* dq,
              float* dk, float* dv, float* dbeta, float* dg_log, float* dS0, void* workspace,
              size_t workspace_bytes, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_chunk(s))) return rc;
  const FwdParams f = make_params(s);
  if (!g_log) dg_log = nullptr;
  const size_t es = esize(s->dtype);
  const size_t nq = (size_t)f.B * f.L * f.H, nx = (size_t)f.B * f.Lx * f.H, nS = (size_t)f.B * f.H * f.DK * f.DV;
  const size_t sz_q = nq * f.DK * es, sz_k = nx * f.DK * es, sz_v = nx * f.DV * es, sz_o = nq * f.DV * es;
  if (nx > 0 && (!q || !k || !v || !beta || !dO || !dq || !dk || !dv || !dbeta)) return DELTA_ERR_NULL_ARG;
  const size_t need = bwd_workspace(f, s->dtype == DELTA_BF16);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DELTA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, S0, dO, dS_final, dq, dk, dv, dS0, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DELTA_ERR_MISALIGNED;
  if (!aligned(beta, 4) || !aligned(g_log, 4) || !aligned(dbeta, 4) || !aligned(dg_log, 4))
    return DELTA_ERR_MISALIGNED;
  const Range in[] = {range(q, q ? sz_q : 0),          range(k, k ? sz_k : 0),
                      range(v, v ? sz_v : 0),          range(beta, beta ? nx * 4 : 0),
                      range(g_log, g_log ? nq * 4 : 0), range(S0, S0 ? nS * 4 : 0),
                      range(dO, dO ? sz_o : 0),         range(dS_final, dS_final ? nS * 4 : 0)};
  const Range out[] = {range(dq, dq ? nq * f.DK * 4 : 0), range(dk, dk ? nx * f.DK * 4 : 0),
                       range(dv, dv ? nx * f.DV * 4 : 0), range(dbeta, dbeta ? nx * 4 : 0),
                       range(dg_log, dg_log ? nq * 4 : 0), range(dS0, dS0 ? nS * 4 : 0),
                       range(workspace, need)};
  constexpr int NO = sizeof(out) / sizeof(out[0]);
  for (int i = 0; i < NO; ++i) {
    for (const Range& r : in)
      if (overlap(out[i], r)) return DELTA_ERR_ALIAS;
    for (int j = i + 1; j < NO; ++j)
      if (overlap(out[i], out[j])) return DELTA_ERR_ALIAS;
  }
  if ((size_t)f.B * f.H == 0) return DELTA_OK;

  const bool bf = s->dtype == DELTA_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((rc = launch_guard())) return rc;
  // the check's flag words take the start of the T region, which the first launch rewrites
  if (validate_on() && f.NT > 0 && (rc = validate_device(beta, nx, g_log, g_log ? nq : 0, ws, st))) return rc;
  if (bwd_scans(f, bf)) {
    // T (bf16), the gate prefix and N; the chunk start states by the forward summary, combine and
    // a chain that stores them; the end-state gradients (and dS0) by the reverse scan; then the
    // per-chunk gradients (and dv) on MFMA
    FwdParams fs = f;
    fs.q = q, fs.k = k, fs.v = v, fs.beta = beta, fs.g_log = g_log, fs.S0 = S0;
    size_t off = 0;
    fs.T = ws;
    off += align_up(t_bytes(f, 2));
    fs.gc = reinterpret_cast<float*>(ws + off);
    off += align_up(gc_bytes(f));
    fs.N = reinterpret_cast<float*>(ws + off);
    off += align_up(t_bytes(f, 4));
    fs.SM = f.P > 1 ? reinterpret_cast<float*>(ws + off) : nullptr;
    off += align_up(sm_bytes(f));
    fs.SMr = f.P > 1 ? reinterpret_cast<float*>(ws + off) : nullptr;  // the reverse scan's summaries
    off += align_up(sm_bytes(f));
    fs.Sst = f.P > 1 ? reinterpret_cast<float*>(ws + off) : nullptr;
    off += align_up(sst_bytes(f));
    void* Sn = ws + off;
    void* Gn = ws + off + align_up(states_bytes(f) / 2);
    void* Gnl = ws + off + 2 * align_up(states_bytes(f) / 2);
    fs.Sn = Sn;
    fs.Snl = nullptr;
    if ((rc = hip_status(delta::launch_intra_chunk(fs, bf, false, st)))) return rc;
    fs.N = nullptr;
    if ((rc = hip_status(delta::launch_scan_phase(fs, bf, delta::SCAN_SUMMARY, st)))) return rc;
    if ((rc = hip_status(delta::launch_scan_phase(fs, bf, delta::SCAN_COMBINE, st)))) return rc;
    if ((rc = hip_status(delta::launch_scan_states(fs, st)))) return rc;
    FwdParams fr = fs;  // the adjoint chain: dO for the values, dS_final in, dS0 out
    fr.v = dO, fr.S0 = dS_final, fr.S_final = dS0, fr.Sn = Gn, fr.Snl = Gnl;
    fr.SM = fs.SMr, fr.SMr = nullptr;
    for (int ph : {delta::SCAN_SUMMARY, delta::SCAN_COMBINE, delta::SCAN_OUTPUTS})
      if ((rc = hip_status(delta::launch_rev_scan(fr, ph, st)))) return rc;
    BwdParams p;
    memset(&p, 0, sizeof(p));
    p.B = f.B, p.L = f.L, p.H = f.H, p.DK = f.DK, p.DV = f.DV, p.nh = f.nh, p.C = f.C, p.Lx = f.Lx, p.NT = f.NT;
    p.scale = f.scale;
    p.q = q, p.k = k, p.v = v, p.beta = beta, p.S0 = S0, p.dO = dO, p.dS_final = dS_final;
    p.dq = dq, p.dk = dk, p.dv = dv, p.dbeta = dbeta, p.dg_log = dg_log, p.dS0 = dS0;
    p.gc = fs.gc;
    p.N = reinterpret_cast<const float*>(ws + align_up(t_bytes(f, 2)) + align_up(gc_bytes(f)));
    p.Snt = Sn, p.Gnt = Gn, p.Gntl = Gnl;
    return hip_status(delta::launch_bwd_chunk_mfma(p, st));
  }
  FwdParams fi = f;  // the intra-chunk launch: T (float32) and the gate prefix
  fi.k = k;
  fi.beta = beta;
  fi.g_log = g_log;
  fi.T = ws;
  fi.gc = reinterpret_cast<float*>(ws + align_up(t_bytes(f, 4)));
  BwdParams p;
  memset(&p, 0, sizeof(p));
  p.B = f.B, p.L = f.L, p.H = f.H, p.DK = f.DK, p.DV = f.DV, p.nh = f.nh, p.C = f.C, p.Lx = f.Lx, p.NT = f.NT;
  p.scale = f.scale;
  p.q = q, p.k = k, p.v = v, p.beta = beta, p.S0 = S0, p.dO = dO, p.dS_final = dS_final;
  p.dq = dq, p.dk = dk, p.dv = dv, p.dbeta = dbeta, p.dg_log = dg_log, p.dS0 = dS0;
  p.T = static_cast<const float*>(fi.T);
  p.gc = fi.gc;
  size_t off = align_up(t_bytes(f, 4)) + align_up(gc_bytes(f));
  p.Pm = reinterpret_cast<float*>(ws + off);
  off += align_up(t_bytes(f, 4));
  p.Sn = reinterpret_cast<float*>(ws + off);
  p.Gn = reinterpret_cast<float*>(ws + off + align_up(states_bytes(f)));
  if (f.NT > 0) {
    if ((rc = hip_status(delta::launch_intra_chunk(fi, bf, true, st)))) return rc;
    if ((rc = hip_status(delta::launch_bwd_phase(p, bf, 3, st)))) return rc;
    if ((rc = hip_status(delta::launch_bwd_phase(p, bf, 0, st)))) return rc;
  }
  // the reverse pass also writes dS0, so it runs when there are no chunks too
  if ((rc = hip_status(delta::launch_bwd_phase(p, bf, 1, st)))) return rc;
  if (f.NT > 0) return hip_status(delta::launch_bwd_phase(p, bf, 2, st));
  return DELTA_OK;
}

namespace {
// A decode step with a scalar gate (g_log) or a per-key-channel one (a_log, KDA).
int run_decode(const delta_shape* s, const void* q, const void* k, const void* v, const float* beta,
               const float* g_log, const float* a_log, float* S, void* O, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (s->L != 1) return DELTA_ERR_BAD_SHAPE;
  if ((size_t)s->B * s->H > 0 && (!q || !k || !v || !beta || !S || !O)) return DELTA_ERR_NULL_ARG;
  const void* ptrs[] = {q, k, v, S, O, a_log};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DELTA_ERR_MISALIGNED;
  if (!aligned(beta, 4) || !aligned(g_log, 4)) return DELTA_ERR_MISALIGNED;
  const size_t es = esize(s->dtype);
  const size_t BH = (size_t)s->B * s->H;
  const Range in[] = {range(q, BH * s->dk * es), range(k, BH * s->n_h * s->dk * es),
                      range(v, BH * s->n_h * s->dv * es), range(beta, BH * s->n_h * 4),
                      range(g_log, g_log ? BH * 4 : 0), range(a_log, a_log ? BH * s->dk * 4 : 0)};
  const Range rS = range(S, BH * s->dk * s->dv * 4), rO = range(O, BH * s->dv * es);
  for (const Range& r : in)
    if (overlap(rS, r) || overlap(rO, r)) return DELTA_ERR_ALIAS;
  if (overlap(rS, rO)) return DELTA_ERR_ALIAS;

  if (BH == 0) return DELTA_OK;
  if ((rc = launch_guard())) return rc;
  if (validate_on() &&
      (rc = validate_small(beta, BH * s->n_h, g_log ? g_log : a_log, g_log ? BH : a_log ? BH * s->dk : 0,
                           static_cast<hipStream_t>(stream))))
    return rc;
  DecodeParams p;
  p.B = s->B;
  p.H = s->H;
  p.DK = s->dk;
  p.DV = s->dv;
  p.nh = s->n_h;
  p.scale = s->scale;
  p.q = q;
  p.k = k;
  p.v = v;
  p.beta = beta;
  p.g_log = g_log;
  p.a_log = a_log;
  p.S = S;
  p.O = O;
  return hip_status(delta::launch_decode(p, s->dtype == DELTA_BF16, static_cast<hipStream_t>(stream)));
}
}  // namespace

int delta_decode(const delta_shape* s, const void* q, const void* k, const void* v, const float* beta,
                 const float* g_log, float* S, void* O, void* stream) {
  return run_decode(s, q, k, v, beta, g_log, nullptr, S, O, stream);
}

int delta_decode_kda(const delta_shape* s, const void* q, const void* k, const void* v, const float* beta,
                     const float* a_log, float* S, void* O, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (s->n_h != 1) return DELTA_ERR_BAD_SHAPE;
  if ((size_t)s->B * s->H > 0 && !a_log) return DELTA_ERR_NULL_ARG;
  return run_decode(s, q, k, v, beta, nullptr, a_log, S, O, stream);
}

int delta_fwd_kda(const delta_shape* s, const void* q, const void* k, const void* v, const float* beta,
                  const float* a_log, const float* S0, void* O, float* S_final, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (s->n_h != 1) return DELTA_ERR_BAD_SHAPE;
  const size_t es = esize(s->dtype);
  const size_t nt = (size_t)s->B * s->L * s->H, BH = (size_t)s->B * s->H;
  if (nt > 0 && (!q || !k || !v || !beta || !a_log || !O)) return DELTA_ERR_NULL_ARG;
  const void* ptrs[] = {q, k, v, a_log, S0, O, S_final};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DELTA_ERR_MISALIGNED;
  if (!aligned(beta, 4)) return DELTA_ERR_MISALIGNED;
  const Range in[] = {range(q, q ? nt * s->dk * es : 0), range(k, k ? nt * s->dk * es : 0),
                      range(v, v ? nt * s->dv * es : 0), range(beta, beta ? nt * 4 : 0),
                      range(a_log, a_log ? nt * s->dk * 4 : 0), range(S0, S0 ? BH * s->dk * s->dv * 4 : 0)};
  const Range ro = range(O, O ? nt * s->dv * es : 0), rs = range(S_final, S_final ? BH * s->dk * s->dv * 4 : 0);
  for (const Range& r : in) {
    if (overlap(ro, r)) return DELTA_ERR_ALIAS;
    if (overlap(rs, r) && !(S0 && S_final == S0 && r.lo == reinterpret_cast<uintptr_t>(S0))) return DELTA_ERR_ALIAS;
  }
  if (overlap(ro, rs)) return DELTA_ERR_ALIAS;
  if (BH == 0 || (s->L == 0 && !S_final)) return DELTA_OK;
  if ((rc = launch_guard())) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (validate_on() && (rc = validate_small(beta, nt, a_log, nt * s->dk, st))) return rc;
  delta::KdaParams p;
  memset(&p, 0, sizeof(p));
  p.B = s->B, p.L = s->L, p.H = s->H, p.DK = s->dk, p.DV = s->dv, p.scale = s->scale;
  p.q = q, p.k = k, p.v = v, p.beta = beta, p.a_log = a_log, p.S0 = S0, p.O = O, p.S_final = S_final;
  return hip_status(delta::launch_kda_fwd(p, s->dtype == DELTA_BF16, st));
}

namespace {
// KDA in chunks: bf16, d_k = d_v = 128, chunk 64, one step per token.  Workspace: T and Aqk (C x C
// bf16 per chunk), K e^{Gc}, K e^{Gc_C - Gc} and Q e^{Gc} (bf16, the layout of k), e^{Gc_C}
// (d_k float32 per chunk), the segment summaries and start states, and each chunk's start state
// (bf16).
bool kda_chunked_shape(const delta_shape* s) {
  return s->dtype == DELTA_BF16 && s->dk == 128 && s->dv == 128 && s->chunk == 64 && s->n_h == 1;
}
size_t kda_tile_bytes(const FwdParams& f) { return (size_t)f.B * f.L * f.H * 128 * 2; }
size_t kda_dc_bytes(const FwdParams& f) { return (size_t)f.B * f.H * f.NT * 128 * 4; }
size_t kda_aqk_bytes(const FwdParams& f) { return (size_t)f.B * f.H * f.NT * delta::KDA_AQK_CHUNK_BYTES; }
size_t kda_chunked_workspace(const FwdParams& f) {
  return align_up(t_bytes(f, 2)) + align_up(kda_aqk_bytes(f)) + 3 * align_up(kda_tile_bytes(f)) + align_up(kda_dc_bytes(f)) +
         align_up(sm_bytes(f)) + align_up(sst_bytes(f));
}
}  // namespace

int delta_fwd_kda_chunked_workspace_bytes(const delta_shape* s, size_t* bytes) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!kda_chunked_shape(s)) return DELTA_ERR_UNSUPPORTED_DIM;
  if (!bytes) return DELTA_ERR_NULL_ARG;
  *bytes = kda_chunked_workspace(make_params(s));
  return DELTA_OK;
}

int delta_fwd_kda_chunked(const delta_shape* s, const void* q, const void* k, const void* v, const float* beta,
                          const float* a_log, const float* S0, void* O, float* S_final, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!kda_chunked_shape(s)) return DELTA_ERR_UNSUPPORTED_DIM;
  const size_t es = 2;
  const size_t nt = (size_t)s->B * s->L * s->H, BH = (size_t)s->B * s->H;
  if (nt > 0 && (!q || !k || !v || !beta || !a_log || !O)) return DELTA_ERR_NULL_ARG;
  const FwdParams f = make_params(s);
  const size_t need = kda_chunked_workspace(f);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DELTA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, a_log, S0, O, S_final, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DELTA_ERR_MISALIGNED;
  if (!aligned(beta, 4)) return DELTA_ERR_MISALIGNED;
  const Range in[] = {range(q, q ? nt * 128 * es : 0), range(k, k ? nt * 128 * es : 0),
                      range(v, v ? nt * 128 * es : 0), range(beta, beta ? nt * 4 : 0),
                      range(a_log, a_log ? nt * 128 * 4 : 0), range(S0, S0 ? BH * 128 * 128 * 4 : 0)};
  const Range ro = range(O, O ? nt * 128 * es : 0), rs = range(S_final, S_final ? BH * 128 * 128 * 4 : 0),
              rw = range(workspace, need);
  for (const Range& r : in) {
    if (overlap(ro, r) || overlap(rw, r)) return DELTA_ERR_ALIAS;
    if (overlap(rs, r) && !(S0 && S_final == S0 && r.lo == reinterpret_cast<uintptr_t>(S0))) return DELTA_ERR_ALIAS;
  }
  if (overlap(ro, rs) || overlap(ro, rw) || overlap(rs, rw)) return DELTA_ERR_ALIAS;
  if (BH == 0 || (s->L == 0 && !S_final)) return DELTA_OK;
  if (s->L == 0) return delta_fwd_kda(s, q, k, v, beta, a_log, S0, O, S_final, stream);  // state passes through
  if ((rc = launch_guard())) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (validate_on() && (rc = validate_small(beta, nt, a_log, nt * 128, st))) return rc;
  char* ws = static_cast<char*>(workspace);
  delta::KdaChunkParams kp;
  memset(&kp, 0, sizeof(kp));
  kp.B = f.B, kp.L = f.L, kp.H = f.H, kp.NT = f.NT, kp.scale = f.scale;
  kp.q = q, kp.k = k, kp.beta = beta, kp.a_log = a_log;
  size_t off = 0;
  kp.T = ws + off;
  off += align_up(t_bytes(f, 2));
  kp.Aqk = ws + off;
  off += align_up(kda_aqk_bytes(f));
  kp.kp = ws + off;
  off += align_up(kda_tile_bytes(f));
  kp.kh = ws + off;
  off += align_up(kda_tile_bytes(f));
  kp.qp = ws + off;
  off += align_up(kda_tile_bytes(f));
  kp.dC = reinterpret_cast<float*>(ws + off);
  off += align_up(kda_dc_bytes(f));
  FwdParams fs = f;
  fs.SM = f.P > 1 ? reinterpret_cast<float*>(ws + off) : nullptr;
  off += align_up(sm_bytes(f));
  fs.Sst = f.P > 1 ? reinterpret_cast<float*>(ws + off) : nullptr;
  fs.k = kp.kp, fs.kh = kp.kh, fs.dC = kp.dC, fs.q = kp.qp, fs.Aqk = kp.Aqk, fs.v = v, fs.T = kp.T;
  fs.beta = beta, fs.S0 = S0, fs.S_final = S_final, fs.O = O;
  if ((rc = hip_status(delta::launch_kda_intra(kp, st)))) return rc;
  for (int ph : {delta::SCAN_SUMMARY, delta::SCAN_COMBINE, delta::SCAN_OUTPUTS})
    if ((rc = hip_status(delta::launch_kda_scan(fs, ph, st)))) return rc;
  return DELTA_OK;
}

int delta_layer_prologue(const delta_shape* s, int32_t width, float eps, const void* xq, const void* xk,
                         const void* xv, const float* wq, const float* wk, const float* wv, void* q, void* k,
                         void* v, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (width < 1 || width > 4) return DELTA_ERR_UNSUPPORTED_DIM;
  if (!(eps >= 0.f)) return DELTA_ERR_BAD_SHAPE;
  const size_t es = esize(s->dtype);
  const size_t rq = (size_t)s->B * s->L * s->H, rkv = rq * s->n_h;
  if ((rkv + 3) / 4 > 0x7fffffffu) return DELTA_ERR_BAD_SHAPE;
  if ((rq > 0 && (!xq || !wq || !q)) || (rkv > 0 && (!xk || !xv || !wk || !wv || !k || !v)))
    return DELTA_ERR_NULL_ARG;
  const void* ptrs[] = {xq, xk, xv, wq, wk, wv, q, k, v};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DELTA_ERR_MISALIGNED;
  const Range in[] = {range(xq, rq * s->dk * es), range(xk, rkv * s->dk * es), range(xv, rkv * s->dv * es),
                      range(wq, (size_t)s->H * s->dk * width * 4), range(wk, (size_t)s->H * s->dk * width * 4),
                      range(wv, (size_t)s->H * s->dv * width * 4)};
  const Range out[] = {range(q, rq * s->dk * es), range(k, rkv * s->dk * es), range(v, rkv * s->dv * es)};
  for (int i = 0; i < 3; ++i) {
    for (const Range& r : in)
      if (overlap(out[i], r)) return DELTA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(out[i], out[j])) return DELTA_ERR_ALIAS;
  }
  if (rkv == 0) return DELTA_OK;  // nothing to do (rq <= rkv)
  if ((rc = launch_guard())) return rc;
  LayerParams p;
  memset(&p, 0, sizeof(p));
  p.B = s->B, p.L = s->L, p.H = s->H, p.DK = s->dk, p.DV = s->dv, p.Lx = s->L * s->n_h, p.width = width;
  p.eps = eps;
  p.xq = xq, p.xk = xk, p.xv = xv, p.wq = wq, p.wk = wk, p.wv = wv, p.q = q, p.k = k, p.v = v;
  return hip_status(delta::launch_layer_prologue(p, s->dtype == DELTA_BF16, static_cast<hipStream_t>(stream)));
}

int delta_layer_prologue_step(const delta_shape* s, int32_t width, float eps, const void* xq, const void* xk,
                              const void* xv, const float* wq, const float* wk, const float* wv, void* conv_q,
                              void* conv_k, void* conv_v, void* q, void* k, void* v, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (s->L != 1) return DELTA_ERR_BAD_SHAPE;
  if (width < 1 || width > 4) return DELTA_ERR_UNSUPPORTED_DIM;
  if (!(eps >= 0.f)) return DELTA_ERR_BAD_SHAPE;
  const size_t es = esize(s->dtype);
  const size_t BH = (size_t)s->B * s->H, nkv = BH * s->n_h, W1 = (size_t)width - 1;
  if (BH > 0 && (!xq || !xk || !xv || !wq || !wk || !wv || !q || !k || !v)) return DELTA_ERR_NULL_ARG;
  if (BH > 0 && W1 > 0 && (!conv_q || !conv_k || !conv_v)) return DELTA_ERR_NULL_ARG;
  const void* ptrs[] = {xq, xk, xv, wq, wk, wv, conv_q, conv_k, conv_v, q, k, v};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DELTA_ERR_MISALIGNED;
  const Range in[] = {range(xq, BH * s->dk * es), range(xk, nkv * s->dk * es), range(xv, nkv * s->dv * es),
                      range(wq, (size_t)s->H * s->dk * width * 4), range(wk, (size_t)s->H * s->dk * width * 4),
                      range(wv, (size_t)s->H * s->dv * width * 4)};
  const Range out[] = {range(q, BH * s->dk * es), range(k, nkv * s->dk * es), range(v, nkv * s->dv * es),
                       range(conv_q, W1 * BH * s->dk * es), range(conv_k, W1 * BH * s->dk * es),
                       range(conv_v, W1 * BH * s->dv * es)};
  constexpr int NO = sizeof(out) / sizeof(out[0]);
  for (int i = 0; i < NO; ++i) {
    for (const Range& r : in)
      if (overlap(out[i], r)) return DELTA_ERR_ALIAS;
    for (int j = i + 1; j < NO; ++j)
      if (overlap(out[i], out[j])) return DELTA_ERR_ALIAS;
  }
  if (BH == 0) return DELTA_OK;
  if ((rc = launch_guard())) return rc;
  LayerParams p;
  memset(&p, 0, sizeof(p));
  p.B = s->B, p.L = 1, p.H = s->H, p.DK = s->dk, p.DV = s->dv, p.Lx = s->n_h, p.width = width;
  p.eps = eps;
  p.xq = xq, p.xk = xk, p.xv = xv, p.wq = wq, p.wk = wk, p.wv = wv, p.q = q, p.k = k, p.v = v;
  p.cq = conv_q, p.ck = conv_k, p.cv = conv_v;
  return hip_status(delta::launch_layer_prologue_step(p, s->dtype == DELTA_BF16, static_cast<hipStream_t>(stream)));
}

int delta_layer_epilogue(const delta_shape* s, float eps, const void* o, const void* g, const float* weight,
                         void* y, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!(eps >= 0.f)) return DELTA_ERR_BAD_SHAPE;
  const size_t es = esize(s->dtype);
  const size_t rows = (size_t)s->B * s->L * s->H;
  if ((rows + 3) / 4 > 0x7fffffffu) return DELTA_ERR_BAD_SHAPE;
  if (rows > 0 && (!o || !g || !weight || !y)) return DELTA_ERR_NULL_ARG;
  const void* ptrs[] = {o, g, weight, y};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DELTA_ERR_MISALIGNED;
  const Range ro = range(o, rows * s->dv * es), rg = range(g, rows * s->dv * es), rw = range(weight, (size_t)s->dv * 4),
              ry = range(y, rows * s->dv * es);
  // y may be o itself (each row is read whole before it is written); no other overlap
  if ((overlap(ry, ro) && y != o) || overlap(ry, rg) || overlap(ry, rw)) return DELTA_ERR_ALIAS;
  if (rows == 0) return DELTA_OK;
  if ((rc = launch_guard())) return rc;
  LayerParams p;
  memset(&p, 0, sizeof(p));
  p.B = s->B, p.L = s->L, p.H = s->H, p.DK = s->dk, p.DV = s->dv, p.Lx = s->L * s->n_h;
  p.eps = eps;
  p.o = o, p.g = g, p.weight = weight, p.y = y;
  return hip_status(delta::launch_layer_epilogue(p, s->dtype == DELTA_BF16, static_cast<hipStream_t>(stream)));
}

const char* delta_strerror(int code) {
  switch (code) {
    case DELTA_OK: return "ok";
    case DELTA_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case DELTA_ERR_BAD_SHAPE: return "bad shape (negative size, n_h < 1, chunk not a multiple of n_h, or too large)";
    case DELTA_ERR_UNSUPPORTED_DIM:
      return "unsupported dimension (dk in {16,32,64,128}, dv a multiple of 16 in [16,256], chunk in "
             "{16,32,48,64}, dtype f32 or bf16)";
    case DELTA_ERR_MISALIGNED: return "a tensor pointer is misaligned (16 bytes; 4 for beta and g_log)";
    case DELTA_ERR_WORKSPACE: return "workspace missing or smaller than delta_fwd_workspace_bytes";
    case DELTA_ERR_ALIAS: return "an output overlaps an input or another output";
    case DELTA_ERR_HIP: return "HIP launch or runtime error";
    case DELTA_ERR_NOALLOC_TOO_LARGE:
      return "delta_fwd_noalloc: the shape needs more workspace than the library's fixed device array "
             "(DELTA_NOALLOC_MAX_BYTES)";
    case DELTA_ERR_BAD_VALUE:
      return "input value outside the contract (non-finite beta, or a NaN or +inf log gate); reported only "
             "with DELTA_VALIDATE=1";
    default: return "unknown error code";
  }
}

}  // extern "C"
