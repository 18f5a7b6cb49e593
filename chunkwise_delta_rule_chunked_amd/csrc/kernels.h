// Launch interface between the C ABI (delta_abi.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace delta {

// One forward problem after validation.  Lx = L * nh expanded positions, NT chunks.
struct FwdParams {
  int B, L, H, DK, DV, nh, C, Lx, NT;
  float scale;
  const void* q;        // [B, L, H, DK]
  const void* k;        // [B, Lx, H, DK]
  const void* v;        // [B, Lx, H, DV]
  const float* beta;    // [B, Lx, H]
  const float* g_log;   // [B, L, H] or nullptr
  const float* S0;      // [B, H, DK, DV] or nullptr
  void* O;              // [B, L, H, DV]
  float* S_final;       // [B, H, DK, DV] or nullptr
  void* T;              // [B, H, NT, C, C]: element type of the inputs, or float for chunk_wy
  float* gc;            // [B, H, NT, C] cumulative in-chunk log gate
  float* W;             // chunk_wy only: [B, H, NT, C, DK]
  float* U;             // chunk_wy only: [B, H, NT, C, DV]
  float* N;             // backward only: [B, H, NT, C, C] (I + A)^-1 in float32, or nullptr
  // sequence split of the inter-chunk pass: P segments of NS chunks (P = 1: no split)
  int P, NS;
  // [B*H, P] segment summaries, each in a slot of DK * (DV + DK) floats: S_loc as float at
  // sloc_index, then, from float offset DV * DK, M in the element type of the inputs at
  // mfrag_index (common.h)
  float* SM;
  float* Sst;           // [B*H, P, DK, DV]: start state of each segment (segments >= 1)
  // KDA chunks (kda_chunk.hip): k holds K e^{Gc}; kh K e^{Gc_C - Gc} (same layout) and dC
  // e^{Gc_C} [B*H, NT, DK], the chunk's decay per key channel; for the outputs, q holds
  // scale Q e^{Gc} and Aqk the causal Q K^T per chunk in the outputs chain's fragment order
  // (KDA_AQK_* below)
  const void* kh;
  const float* dC;
  const void* Aqk;
  // backward only: the summary launch also writes each segment's transition map transposed, in
  // the M part of slot P - 1 - seg of these summaries (the reverse scan's, whose segments are
  // numbered from the end and whose transition maps are the forward's transposed)
  float* SMr;
  // backward scans only: [B*H, NT, DV, DK] in the element type of the inputs, each chunk's start
  // state (forward chain) or end-state gradient (reverse chain), transposed; the reverse chain
  // also stores the rounding residual of each gradient (G - Sn, rounded) at Snl
  void* Sn;
  void* Snl;
};

struct DecodeParams {
  int B, H, DK, DV, nh;
  float scale;
  const void* q;        // [B, 1, H, DK]
  const void* k;        // [B, nh, H, DK]
  const void* v;        // [B, nh, H, DV]
  const float* beta;    // [B, nh, H]
  const float* g_log;   // [B, 1, H] or nullptr
  const float* a_log;   // [B, 1, H, DK] per-key-channel log decay (KDA) or nullptr
  float* S;             // [B, H, DK, DV], in place
  void* O;              // [B, 1, H, DV]
};

// KDA forward over a sequence (kda.hip): n_h = 1, a decay per key channel.
struct KdaParams {
  int B, L, H, DK, DV;
  float scale;
  const void* q;        // [B, L, H, DK]
  const void* k;        // [B, L, H, DK]
  const void* v;        // [B, L, H, DV]
  const float* beta;    // [B, L, H]
  const float* a_log;   // [B, L, H, DK] log alpha per key channel
  const float* S0;      // [B, H, DK, DV] or nullptr
  void* O;              // [B, L, H, DV]
  float* S_final;       // [B, H, DK, DV] or nullptr; may be S0
};

// KDA forward in chunks (kda_chunk.hip): bf16, d_k = d_v = 128, chunk 64, one step per token.
// KDA in chunks, chunk 64: Aqk's lower triangle as the outputs chain reads it, per chunk
// KDA_AQK_FRAGS fragments of 64 lanes x 16 bytes.  Fragment f = (bb, kp) in the order (0,0) (1,0)
// (2,0) (2,1) (3,0) (3,1) (token block bb of 16 rows, 32-token pair kp <= bb / 2); lane (g, m)
// holds Aqk[16 bb + m][32 kp + 4 g .. + 3] and then Aqk[16 bb + m][32 kp + 16 + 4 g .. + 3] (zeros
// past the diagonal), bf16.
constexpr int KDA_AQK_FRAGS = 6;
constexpr int KDA_AQK_CHUNK_BYTES = KDA_AQK_FRAGS * 64 * 16;
__host__ __device__ constexpr int kda_aqk_block(int f) { return f == 0 ? 0 : f == 1 ? 1 : f < 4 ? 2 : 3; }
__host__ __device__ constexpr int kda_aqk_pair(int f) { return (f == 3 || f == 5) ? 1 : 0; }

struct KdaChunkParams {
  int B, L, H, NT;
  float scale;
  const void* q;        // [B, L, H, 128] bf16
  const void* k;        // [B, L, H, 128] bf16
  const float* beta;    // [B, L, H]
  const float* a_log;   // [B, L, H, 128] log alpha per key channel
  // per chunk, written by the intra launch: T [B*H, NT, C, C] bf16, Aqk (KDA_AQK_* below); K e^{Gc},
  // K e^{Gc_C - Gc} and scale Q e^{Gc} in the layout of k [B, L, H, 128] bf16; e^{Gc_C}
  // [B*H, NT, 128] float32
  void* T;
  void* Aqk;
  void* kp;
  void* kh;
  void* qp;
  float* dC;
};

// One backward problem after validation (shape fields as in FwdParams).
struct BwdParams {
  int B, L, H, DK, DV, nh, C, Lx, NT;
  float scale;
  const void* q;          // [B, L, H, DK]
  const void* k;          // [B, Lx, H, DK]
  const void* v;          // [B, Lx, H, DV]
  const float* beta;      // [B, Lx, H]
  const float* S0;        // [B, H, DK, DV] or nullptr
  const void* dO;         // [B, L, H, DV], element type of the inputs
  const float* dS_final;  // [B, H, DK, DV] or nullptr (zero)
  float* dq;              // [B, L, H, DK]
  float* dk;              // [B, Lx, H, DK]
  float* dv;              // [B, Lx, H, DV]
  float* dbeta;           // [B, Lx, H]
  float* dg_log;          // [B, L, H] or nullptr (ungated)
  float* dS0;             // [B, H, DK, DV] or nullptr
  const float* T;         // [B*H, NT, C, C] float32, from the intra-chunk launch
  const float* gc;        // [B*H, NT, C]
  float* Pm;              // [B*H, NT, C, C] Q K^T * Gam on and below the diagonal (Q scaled)
  float* Sn;              // [B*H, NT, DK, DV] start state of each chunk
  float* Gn;              // [B*H, NT, DK, DV] state gradient at the end of each chunk
  const float* N;         // [B*H, NT, C, C] (I + A)^-1 float32 (the MFMA per-chunk kernel)
  // the MFMA per-chunk kernel: Sn and Gn as bf16 [B*H, NT, DV, DK] (transposed), from the scans,
  // and Gn's rounding residual (G' = Gnt + Gntl to about 16 bits)
  const void* Snt;
  const void* Gnt;
  const void* Gntl;
};

// The layer steps around the mixer (layer.hip).
struct LayerParams {
  int B, L, H, DK, DV, Lx, width;
  float eps;
  const void *xq, *xk, *xv;       // prologue inputs [B, L, H, DK], [B, Lx, H, DK], [B, Lx, H, DV]
  const float *wq, *wk, *wv;      // [H * d, width] conv filters
  void *q, *k, *v;                // prologue outputs, shapes as the inputs
  void *cq, *ck, *cv;             // decode step: filter states [B, width - 1, H, d], in/out
  const void* o;                  // epilogue: mixer output [B, L, H, DV]
  const void* g;                  // gate projection [B, L, H, DV]
  const float* weight;            // [DV]
  void* y;                        // [B, L, H, DV]
};

// Each returns hipSuccess or the launch error.  `bf16` selects the element type of
// q/k/v/O (true: bfloat16, false: float32).
hipError_t launch_intra_chunk(const FwdParams& p, bool bf16, bool t_as_float, hipStream_t st);
hipError_t launch_wy_factors(const FwdParams& p, bool bf16, hipStream_t st);
// The three launches of the inter-chunk pass (see chunk_scan.hip): segment summaries,
// segment start states, outputs.  The first two do nothing when P == 1.
enum { SCAN_SUMMARY = 0, SCAN_COMBINE = 1, SCAN_OUTPUTS = 2 };
hipError_t launch_scan_phase(const FwdParams& p, bool bf16, int phase, hipStream_t st);
// Summary launch for bf16 inputs, d_k = d_v = 128, chunk 64 (scan_summary.hip).
bool scan_summary_fast_applies(const FwdParams& p, bool bf16);
hipError_t launch_scan_summary_fast(const FwdParams& p, hipStream_t st);
hipError_t launch_scan_summary_fast_kda(const FwdParams& p, hipStream_t st);  // KDA in chunks
// KDA in chunks: the chain on the value columns from each segment's start state forming O (and
// S_final), from the intra kernel's K+, Kh, Q+, T, Aqk and e^{Gc_C}
hipError_t launch_scan_outputs_kda(const FwdParams& p, hipStream_t st);
// The backward pass's state scans on the inter-chunk machinery, for bf16 inputs with
// d_k = d_v = 128 and chunk 64 (chunk_scan.hip).  After the forward summary and combine,
// launch_scan_states runs the forward chain writing each chunk's start state to p.Sn.  The
// reverse scan takes p.v = dO, p.S0 = dS_final, p.S_final = dS0, p.Sn = end-state gradients, and
// runs the same three phases (the combine unchanged) with segments numbered from the end.
bool bwd_scans_apply(const FwdParams& p, bool bf16);
hipError_t launch_scan_states(const FwdParams& p, hipStream_t st);
hipError_t launch_rev_scan(const FwdParams& p, int phase, hipStream_t st);
// KDA in chunks: the intra launch (kda_chunk.hip), the scan's summary and state-storing chain in
// KDA mode (chunk_scan.hip; the combine is the forward's), the output launch.
hipError_t launch_kda_intra(const KdaChunkParams& p, hipStream_t st);
hipError_t launch_kda_scan(const FwdParams& p, int phase, hipStream_t st);
// Backward launches (backward.hip), in order after launch_intra_chunk with float T:
// 3 Q K^T * Gam per chunk, 0 chunk start states, 1 end-of-chunk state gradients (and dv, dS0),
// 2 per-chunk gradients.
hipError_t launch_bwd_phase(const BwdParams& p, bool bf16, int phase, hipStream_t st);
// Per-chunk gradients on MFMA for bf16 inputs, d_k = d_v = 128, chunk 64 (backward_mfma.hip), in
// place of phase 2; reads N (float32, from the intra-chunk launch) instead of recomputing it.
bool bwd_chunk_mfma_applies(const BwdParams& p, bool bf16);
hipError_t launch_bwd_chunk_mfma(const BwdParams& p, hipStream_t st);
hipError_t launch_layer_prologue(const LayerParams& p, bool bf16, hipStream_t st);
hipError_t launch_layer_epilogue(const LayerParams& p, bool bf16, hipStream_t st);
hipError_t launch_layer_prologue_step(const LayerParams& p, bool bf16, hipStream_t st);
hipError_t launch_decode(const DecodeParams& p, bool bf16, hipStream_t st);
hipError_t launch_kda_fwd(const KdaParams& p, bool bf16, hipStream_t st);
// Opt-in input check (validate.hip): beta finite, log gates finite or -inf.  Writes one flag word
// per workgroup (VALIDATE_BLOCKS words) at `flags`.
constexpr int VALIDATE_BLOCKS = 128;
hipError_t launch_validate(const float* beta, long nbeta, const float* glog, long ngate, unsigned* flags,
                           hipStream_t st);

}  // namespace delta
