// Host-side launch interface between the C ABI (ssd_api.hip) and the kernel files.
// Every launcher assumes its arguments were validated by the API layer.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

enum { DT_F32 = 0, DT_BF16 = 1 };

struct FwdArgs {
  int B, L, H, P, N, G, Q, nc;
  int dtype;
  const void* x;
  const void* dt;
  const float* dt_bias;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* D;          // may be null
  const void* z;           // gate, may be null
  float dt_lo, dt_hi;      // clamp of dt' when clamp != 0
  int clamp;
  const float* init;       // may be null
  void* y;
  float* final_state;      // may be null
  float* dtp;              // workspace (B, H, nc, Q)
  float* dAcs;             // workspace (B, H, nc, Q)
  float* states;           // workspace (B, nc, H, P, N)
  void* prev16;            // bf16 only: the states entering each chunk rounded to bf16, (B, nc, H, P, N),
                           // written by state_passing and read by chunk_scan; null: fp32 states
  int keep_f32_states;     // with prev16: also keep the fp32 states entering each chunk (backward)
  float* cb;               // workspace: C B^T sub-tiles per (b, c, g), see cb_block (fp32, and
                           // bf16 with many heads per group); null: chunk_state does not form them
  float* cbT;              // backward (fp32): the same blocks in bwd_dxdb's layout (cb_block TRANS);
                           // null: not formed
  int heads_per_block;     // chunk_scan: heads sharing one C B^T evaluation (divides H / G); for
                           // scan_variant 3 the heads of a workgroup's slice
  int scan_variant;        // chunk_scan decomposition: 1 = 64-row blocks, 2 = whole chunks, 3 = a
                           // chunk of one group and a slice of its heads (bf16, chunk 256, P64 N128)
  int rows_group;          // row blocks: units per dispatch group on an XCD (0: all of one class first)
  hipEvent_t ev0, ev1;     // timing: start / stop events of the next launch (or null), recorded
                           // by the dispatch itself (hipExtLaunchKernelGGL), so they time the
                           // kernel alone, as a profiler's kernel trace does
  int state_from_start;    // chunk_state weights exp(dAcs_i) instead of exp(last - dAcs_i) dt'_i,
                           // reading dt' and the cumsum instead of computing them
  int passing_reverse;     // state_passing from the last chunk to the first
  // segmented chunk states (chunk_state_seg): prev16 holds the states each segment alone carried
  // into its chunks (none for a segment's first chunk); chunk_scan adds exp(cdec) hin16
  int seg_len;             // chunks per segment, 0 = no segments
  const void* hin16;       // (B, nseg, H, P, N) bf16: the state entering each segment
  const float* cdec;       // (B, H, nc): exponent of the decay from the segment start to chunk c
};

// The segmented chunk-state launch: heads per workgroup, chunks per segment, and its outputs.
struct SegArgs {
  int hs, SL, nseg;
  float* E;                // (B, nseg, H, P, N) fp32: each segment's end state from a zero start
  float* segdec;           // (B, H, nseg): the segment's total decay exponent
  float* cdec;             // (B, H, nc)
};

// Backward pass (ssd_bwd): the forward's workspace regions plus the gradient buffers.
struct BwdArgs {
  FwdArgs f;               // forward sizes, inputs and recomputed intermediates
  const void* dy;          // (B, L, H, P) dtype: gradient of the pre-gate output
  float* gstates;          // (B, nc, H, P, N): gradient of the state leaving each chunk
  int hs_dxdb = 1;         // heads per slice: bwd_dxdb sums dB over a slice of hs_dxdb consecutive
                           // heads of one group in registers (1, or 4 for bf16; divides H / G)
  int hs_dc = 1;           // the same for bwd_dc and dC
  float* dBh;              // (B, L, H / hs_dxdb, N) per-slice dB
  float* dCh;              // (B, L, H / hs_dc, N) per-slice dC
  float* ddir;             // (B, H, nc, Q) direct d(dt') term
  float* dSa;              // (B, H, nc, Q) anti-causal part of d(dAcs)
  float* dSc;              // (B, H, nc, Q) causal part of d(dAcs)
  float* Ub;               // (B, H, nc, Q) state-input term
  float* pA;               // (B, nc, H) partial dA
  float* pbias;            // (B, nc, H) partial d dt_bias
  float* pD;               // (B, nc * Q/64, H, P) partial dD
  void* dx;
  void* ddt;
  void* dB;
  void* dC;
  float* ddt_bias;
  float* dA;
  float* dD;               // may be null
};

struct GateArgs {
  int64_t n;               // elements
  int dtype;
  const void* dout;
  const void* z;
  const void* ypre;
  void* dy;
  void* dz;
  hipEvent_t ev0, ev1;
};

struct StepArgs {
  int B, H, P, N, G;
  int dtype;
  float* state;
  const void* x;
  const void* dt;
  const float* dt_bias;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* D;
  const void* z;
  float dt_lo, dt_hi;
  int clamp;
  void* y;
  hipEvent_t ev0, ev1;     // timing events recorded by the dispatch (or null)
};

// Causal depthwise conv1d + SiLU over xBC = [x | B | C] channels (Dc = dx + 2 dbc).
struct ConvArgs {
  int B, L, Dc, dx, dbc, K;
  int dtype;
  const void* xbc;         // (B, L, Dc), or (B, Dc) for the decode step
  const float* w;          // (Dc, K)
  const float* bias;       // (Dc) or null
  const void* state_in;    // (B, K-1, Dc) or null (zeros); the decode step updates it in place
  void* state_out;         // (B, K-1, Dc) or null; may equal state_in
  void* x;                 // (B, L, dx)
  void* Bo;                // (B, L, dbc)
  void* Co;                // (B, L, dbc)
  int segment;             // conv1d_silu tokens per thread (multiple of 16); 0 = sized to the chip
};

// true when a kernel instantiation exists for (dtype, P, N)
bool shape_supported(int dtype, int P, int N);

hipError_t launch_chunk_state(const FwdArgs& a, hipStream_t s);
hipError_t launch_state_passing(const FwdArgs& a, hipStream_t s);
// forward only: chunk states and state passing in one launch, one workgroup per (b, h, ps
// headdim rows); supported(a, ps): an instantiation exists for (dtype, P, N, ps)
bool chunk_state_seq_supported(const FwdArgs& a, int ps);
hipError_t launch_chunk_state_seq(const FwdArgs& a, int ps, hipStream_t s);
hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t s);
// scan_variant 3 (chunk_scan_group.hip): an instantiation exists for these sizes
bool chunk_scan_group_supported(int dtype, int P, int N, int Q);
// segmented chunk states (chunk_state_seg.hip), hs heads per workgroup
bool chunk_state_seg_supported(int dtype, int P, int N, int Q, int hs);
hipError_t launch_chunk_state_seg(const FwdArgs& a, const SegArgs& sg, hipStream_t s);
hipError_t launch_chunk_scan_group(const FwdArgs& a, int hs, hipStream_t s);
hipError_t launch_ssd_step(const StepArgs& a, hipStream_t s);
hipError_t launch_bwd_dxdb(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dc(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_finalize(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_reduce(const BwdArgs& a, hipStream_t s);
hipError_t launch_gate_bwd(const GateArgs& a, hipStream_t s);
hipError_t launch_conv1d_silu(const ConvArgs& a, hipStream_t s);

// Gated RMSNorm of the scan output (gated_norm.hip).
struct NormArgs {
  int64_t tokens;          // B * L
  int H, P, norm_heads;    // norm_heads divides H
  int dtype;
  const void* y;           // (tokens, H, P)
  const void* z;           // same shape, or null (no gate)
  const float* weight;     // (H * P)
  void* out;               // same shape; y itself or disjoint from y and z
  float eps;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;   // optional dispatch events
};
hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t s);
hipError_t launch_conv1d_silu_step(const ConvArgs& a, hipStream_t s);

}  // namespace ssd

// (dtype, P, N) instantiation lists.  fp32 MFMA contracts over N in steps of 4, bf16 in
// steps of 32, hence the different dstate sets.
#define SSD_FOR_EACH_SHAPE(X) \
  X(float, 16, 16) X(float, 16, 32) X(float, 16, 64) \
  X(float, 32, 16) X(float, 32, 32) X(float, 32, 64) \
  X(float, 64, 16) X(float, 64, 32) X(float, 64, 64) \
  X(__bf16, 16, 32) X(__bf16, 16, 64) X(__bf16, 16, 128) \
  X(__bf16, 32, 32) X(__bf16, 32, 64) X(__bf16, 32, 128) \
  X(__bf16, 64, 32) X(__bf16, 64, 64) X(__bf16, 64, 128)

#define SSD_DTYPE_CODE_float 0
#define SSD_DTYPE_CODE___bf16 1
