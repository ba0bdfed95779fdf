// C ABI of libssd.so: argument validation, workspace carving and kernel launch order.
// Declarations and the contract live in include/ssd.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>
#include <stdlib.h>

#include "ssd.h"
#include "ssd_tuning.h"
#include "ssd_launch.h"

namespace {

constexpr size_t kRegionAlign = 256;

size_t align_up(size_t v) { return (v + kRegionAlign - 1) / kRegionAlign * kRegionAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_bytes(int dtype) { return dtype == SSD_F32 ? 4 : 2; }

// Shape checks common to both entry points.  Returns SSD_OK or the error.
ssd_status_t check_dims(const ssd_dims_t* d, bool need_seqlen) {
  if (!d) return SSD_ERR_INVALID_ARG;
  if (d->batch < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 || d->ngroups < 1) return SSD_ERR_INVALID_ARG;
  if (need_seqlen && d->seqlen < 0) return SSD_ERR_INVALID_ARG;
  if (d->nheads % d->ngroups != 0) return SSD_ERR_INVALID_ARG;
  // dt clamp: off when both bounds are 0, else 0 <= dt_min <= dt_max with dt_max > 0 (NaN fails)
  if (!(d->dt_min >= 0.f) || !(d->dt_max >= d->dt_min)) return SSD_ERR_INVALID_ARG;
  if (d->dt_max == 0.f && d->dt_min != 0.f) return SSD_ERR_INVALID_ARG;
  if (d->dtype != SSD_F32 && d->dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
  if (!ssd::shape_supported(d->dtype, (int)d->headdim, (int)d->dstate)) return SSD_ERR_UNSUPPORTED;
  // 32-bit index arithmetic bounds of the launchers (grid sizes, per-sequence offsets)
  if (d->batch > 65535 || d->nheads > 65535 || d->seqlen > (int64_t)1 << 30) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

bool chunk_ok(int q) { return q == 64 || q == 128 || q == 256; }

struct WsLayout {
  size_t dtp_off, dacs_off, states_off, cb_off, prev16_off, segs_off, total;
};

// bf16 only: the segmented chunk-state path's per-(b, h) exponents, segment totals then the
// exponents from each chunk's segment start, 2 x (B, H, nc) fp32 (at most nc segments)
size_t segs_bytes(const ssd_dims_t* d, int Q) {
  if (d->dtype != SSD_BF16) return 0;
  const int64_t nc = (d->seqlen + Q - 1) / Q;
  return 2 * align_up((size_t)d->batch * d->nheads * nc * sizeof(float));
}

// bf16 only: the states entering each chunk rounded to bf16, (B, nc, H, P, N)
size_t prev16_bytes(const ssd_dims_t* d, int Q) {
  if (d->dtype != SSD_BF16) return 0;
  const int64_t nc = (d->seqlen + Q - 1) / Q;
  return align_up((size_t)d->batch * nc * d->nheads * d->headdim * d->dstate * 2);
}

// C B^T formed once per group by chunk_state (cb_block) and read by every head's scan: always
// for fp32; for bf16 when a group has at least 20 heads.  For bf16 the scan can also form it
// itself from the bf16 rows, and the blocks (16 KB of fp32 per 64 x 64 block) cost chunk_state
// more than they save the scan below that: measured on MI355X, 32 heads per group (B8 L4096
// H32 N128) 0.341 -> 0.320 ms per forward, 10 heads per group (B2 L16384 H80 G8) 0.795 ->
// 0.819 ms.
bool cb_shared(const ssd_dims_t* d) { return d->dtype == SSD_F32 || d->nheads / d->ngroups >= 20; }

// the C B^T sub-tile blocks cb_block writes, (B, nc, G, nrb (nrb + 1) / 2) x 16 KB (fp32)
size_t cb_bytes(const ssd_dims_t* d, int Q) {
  if (!cb_shared(d)) return 0;
  const int64_t nc = (d->seqlen + Q - 1) / Q, nrb = Q / 64;
  return align_up((size_t)d->batch * nc * d->ngroups * (nrb * (nrb + 1) / 2) * 16 * 256 * sizeof(float));
}

WsLayout ws_layout(const ssd_dims_t* d, int Q) {
  const int64_t nc = (d->seqlen + Q - 1) / Q;
  WsLayout w;
  const size_t cum = align_up((size_t)d->batch * d->nheads * nc * Q * sizeof(float));
  const size_t st = align_up((size_t)d->batch * nc * d->nheads * d->headdim * d->dstate * sizeof(float));
  w.dtp_off = 0;
  w.dacs_off = cum;
  w.states_off = 2 * cum;
  w.cb_off = 2 * cum + st;
  w.prev16_off = w.cb_off + cb_bytes(d, Q);
  w.segs_off = w.prev16_off + prev16_bytes(d, Q);
  w.total = w.segs_off + segs_bytes(d, Q);
  return w;
}

// Is p device memory usable by the current device?
bool device_ptr_ok(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error the failed query leaves
    return false;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (attr.type == hipMemoryTypeDevice) return attr.device == dev;
  return attr.type == hipMemoryTypeManaged;
}

// Launch choices: pure functions of the sizes and the caller's options (NULL = built-in).
const ssd_launch_opts_t kBuiltin{};
const ssd_launch_opts_t& opts_or_builtin(const ssd_launch_opts_t* o) { return o ? *o : kBuiltin; }

// Chunk states.  Three paths:
//  1: chunk_state per (b, c, h) in parallel, then the sequential state_passing launch;
//  2: one pass per (b, h, headdim slice) walking the chunks in order with the state in registers
//     (no per-chunk states in memory);
//  3: segments of SL chunks per (b, group, slice of hs heads), each from a zero state, combined
//     by state_passing over segments, the scan adding each segment's incoming state (needs the
//     scan's group form, which applies that correction).
struct StatePath {
  int path = 1;
  int ps = 0;            // path 2: headdim rows per workgroup
  int hs = 0, SL = 0;    // path 3: heads per workgroup, chunks per segment
};

int seg_heads(int hpg, int want) {
  if (want > 0) return ssd::chunk_state_seg_supported(ssd::DT_BF16, 64, 128, 256, want) && hpg % want == 0 ? want : 0;
  for (int hs : {5, 4, 2, 1})
    if (hpg % hs == 0) return hs;
  return 0;
}

// Built-in choice, measured on MI355X (bf16 P64 N128): one pass from B H >= 256 (B8 L4096 H32
// forward 0.320 -> 0.277 ms, B16 L2048 0.338 -> 0.299, B8 L1024 0.092 -> 0.082, B8 L4096 chunk
// 128 0.378 -> 0.344); below that the one-pass chains are too few for 256 CUs (B4 L4096 H32 0.163
// against 0.172 ms for two launches; B2 L16384 H80 G8 0.793 against 0.823), and segments take
// over where the scan's group form applies (below); fp32 keeps two launches (B4 L1024 H24 0.0695
// against 0.0765 ms at 32-row slices, B16 L1024 H24 0.230 against 0.228 at whole rows).
StatePath pick_state_path(int dtype, int64_t B, int64_t H, int64_t G, int P, int N, int Q, int nc, bool forward_only,
                          int scan_variant, const ssd_launch_opts_t& o) {
  StatePath sp;
  if (o.state_path == 1 || !forward_only) return sp;
  ssd::FwdArgs a{};
  a.dtype = dtype;
  a.P = P;
  a.N = N;
  a.Q = Q;
  if (o.state_path == 3) {
    // segments: SL chunks each, at least two so that the segment states fit the chunk-state region
    const int hs = seg_heads((int)(H / G), o.state_heads);
    if (hs > 0 && scan_variant == 3 && ssd::chunk_state_seg_supported(dtype, P, N, Q, hs)) {
      const int SL = o.state_chunks > 0 ? o.state_chunks : 8;
      const int nseg = (nc + SL - 1) / SL;
      if (SL >= 2 && 3 * nseg <= 2 * nc) {
        sp.path = 3;
        sp.hs = hs;
        sp.SL = SL;
        return sp;
      }
    }
    return sp;
  }
  if (o.state_path == 2) {
    const int ps = o.state_slice > 0 ? o.state_slice : P;
    if (ssd::chunk_state_seq_supported(a, ps)) {
      sp.path = 2;
      sp.ps = ps;
    }
    return sp;
  }
  if (dtype != ssd::DT_BF16 || P != 64 || N != 128) return sp;
  // enough chains for the one pass: it is kept except on long sequences whose groups have at
  // least four slices of heads sharing B, where segments win.  Measured on MI355X (forward, ms,
  // one pass / segments): B8 L4096 H32 G1 0.207 / 0.192, B16 L4096 H32 0.420 / 0.373, B8 L8192
  // H32 0.417 / 0.382; kept: B16 L2048 H32 0.207 / 0.236, B8 L1024 H32 0.066 / 0.097, B4 L4096
  // H64 G8 (two slices per group) 0.228 / 0.253
  const int hs_seg = seg_heads((int)(H / G), o.state_heads);
  const bool seg_long = hs_seg > 0 && scan_variant == 3 && ssd::chunk_state_seg_supported(dtype, P, N, Q, hs_seg) &&
                        nc >= 16 && (H / G) / hs_seg >= 4;
  if (B * H >= 256 && !seg_long) {
    if (ssd::chunk_state_seq_supported(a, 64)) {
      sp.path = 2;
      sp.ps = 64;
    }
    return sp;
  }
  // fewer chains than CUs (or the long sequences above): segments, sized for at least 256
  // workgroups.  Measured on MI355X, bf16
  // B2 L16384 H80 G8 (64 chunks, 5 heads per workgroup): segments of 8 / 4 / 2 chunks 0.701 /
  // 0.724 / 0.752 ms per forward against 0.808 for two launches (chunk_state 256 + state_passing
  // 85 us -> 209 + 11 us; the scan's correction costs it 404 -> 445 us)
  // (segment sizes given in the options apply here too)
  const int hs = seg_heads((int)(H / G), o.state_heads);
  if (hs > 0 && scan_variant == 3 && ssd::chunk_state_seg_supported(dtype, P, N, Q, hs) && nc >= 3) {
    const long per_seg = B * G * ((H / G) / hs);                 // workgroups per segment index
    const int nseg_want = (int)((256 + per_seg - 1) / per_seg);
    int SL = o.state_chunks > 0 ? o.state_chunks : (nc + nseg_want - 1) / nseg_want;
    if (SL < 2) SL = 2;
    if (3 * ((nc + SL - 1) / SL) <= 2 * nc) {
      sp.path = 3;
      sp.hs = hs;
      sp.SL = SL;
    }
  }
  return sp;
}

// Row-block dispatch groups of 16 units per XCD: measured on MI355X, bf16 B2 L16384 H80 G8
// chunk_scan 514 -> 432 us (the row blocks of a unit re-read its x tiles and entering state
// from L2 instead of HBM); B8 L4096 H32 and fp32 B4 L1024 unchanged within noise.
int pick_rows_group(const ssd_launch_opts_t& o) { return o.rows_group > 0 ? o.rows_group : 16; }

// chunk_scan decomposition.  Two: 64-row blocks (many small workgroups: x tiles and the
// carried state are re-read per row block, from L2 when dispatched in groups) and whole chunks
// (every input and output moves once).  Row blocks for both dtypes: measured on MI355X, fp32
// B4 L1024 H24 39 us against 68 us for whole chunks; bf16 B8 L4096 H32 N128 191 us against
// 208 us (bf16 B2 L16384 H80 G8: 545 us against 519 us, the one shape measured where whole
// chunks win).
// The group form (a workgroup per chunk, group and slice of heads, C B^T formed once per slice)
// wherever it is instantiated (bf16, chunk 256, P64 N128): measured on MI355X, bf16 B2 L16384 H80
// G8 chunk_scan 456 -> 398 us, B8 L4096 H32 on par (162 us) with chunk_state_seq 122 -> 101 us,
// since no C B^T blocks are formed for the scan to read.
int pick_scan_variant(const ssd_dims_t* d, int Q, const ssd_launch_opts_t& o) {
  const bool group = ssd::chunk_scan_group_supported(d->dtype, (int)d->headdim, (int)d->dstate, Q);
  if (o.scan_variant == 1 || o.scan_variant == 2 || (o.scan_variant == 3 && group)) return o.scan_variant;
  return group ? 3 : 1;
}

// Heads of one group sharing one C B^T evaluation inside a workgroup; more heads per workgroup
// amortise it further but leave fewer workgroups to fill 256 CUs.
int pick_heads_per_block(int B, int nc, int H, int G, int variant, const ssd_launch_opts_t& o) {
  static const int kChoices[] = {2, 1};  // instantiated head-block sizes
  const int hpg = H / G;
  if (variant == 3) {
    // a workgroup per (b, c, g, slice of heads): any slice size that divides the group.  Built-in:
    // the largest slice of at most 16 heads that still leaves a workgroup per CU (C B^T once per
    // slice; a workgroup fills a CU).  Measured on MI355X: B2 L16384 H80 G8 slices of 10 / 5 / 2
    // heads 398 / 433 / 533 us; B8 L4096 H32 slices of 16 / 8 / 4 / 2 163 / 162 / 185 / 222 us.
    if (o.heads_per_block > 0 && hpg % o.heads_per_block == 0) return o.heads_per_block;
    const long units = (long)B * nc * G;
    for (int hs = hpg < 16 ? hpg : 16; hs > 1; --hs)
      if (hpg % hs == 0 && units * (hpg / hs) >= 256) return hs;
    return 1;
  }
  if (o.heads_per_block > 0) {
    for (int hb : kChoices)
      if (hb == o.heads_per_block && hpg % hb == 0) return hb;
  }
  // row blocks: one head per workgroup (a second head's accumulators would halve occupancy)
  if (variant == 1) return 1;
  // whole chunks: the largest head block that still leaves enough workgroups
  const long per_head = (long)B * nc * G;
  const long min_blocks = o.min_blocks > 0 ? o.min_blocks : 512;
  for (int hb : kChoices)
    if (hpg % hb == 0 && per_head * (hpg / hb) >= min_blocks) return hb;
  return 1;
}

ssd_status_t fwd_impl(const ssd_dims_t* dims, const void* x, const void* dt, const float* dt_bias,
                      const float* A, const void* B, const void* C, const float* D, const void* z,
                      int chunk_size, const float* initial_state, void* y, float* final_state, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, const ssd_launch_opts_t* opts, hipEvent_t* ev,
                      bool own_scratch = false) {
  const ssd_launch_opts_t& o = opts_or_builtin(opts);
  ssd_status_t st = check_dims(dims, true);
  if (st != SSD_OK) return st;
  if (!chunk_ok(chunk_size)) return SSD_ERR_UNSUPPORTED;
  if (dims->batch == 0) return SSD_OK;
  const bool has_seq = dims->seqlen > 0;
  const size_t eb = elem_bytes(dims->dtype);

  // required pointers and alignment
  if (has_seq) {
    if (!x || !dt || !dt_bias || !A || !B || !C || !y) return SSD_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16)) return SSD_ERR_INVALID_ARG;
    if (!aligned(dt, eb) || !aligned(dt_bias, 4) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
        (z && !aligned(z, eb)))
      return SSD_ERR_INVALID_ARG;
  }
  if ((initial_state && !aligned(initial_state, 16)) || (final_state && !aligned(final_state, 16)))
    return SSD_ERR_INVALID_ARG;
  const WsLayout wl = ws_layout(dims, chunk_size);
  if (has_seq) {
    if (!workspace || workspace_bytes < wl.total) return SSD_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return SSD_ERR_INVALID_ARG;
  }
  // every pointer must be device memory of the current device
  // (the library's own scratch array is a module global, not a runtime allocation: not queried)
  const void* ptrs[] = {x,  dt, dt_bias, A, B, C, D, has_seq ? z : nullptr, initial_state, y, final_state,
                        has_seq && !own_scratch ? workspace : nullptr};
  for (const void* p : ptrs)
    if (p && !device_ptr_ok(p)) return SSD_ERR_DEVICE_PTR;

  // timing events cannot be recorded into a graph capture on this runtime: refuse up front
  if (ev) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return SSD_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) return SSD_ERR_UNSUPPORTED;
  }

  ssd::FwdArgs a;
  a.B = (int)dims->batch;
  a.L = (int)dims->seqlen;
  a.H = (int)dims->nheads;
  a.P = (int)dims->headdim;
  a.N = (int)dims->dstate;
  a.G = (int)dims->ngroups;
  a.Q = chunk_size;
  a.nc = (int)((dims->seqlen + chunk_size - 1) / chunk_size);
  a.dtype = dims->dtype;
  a.x = x;
  a.dt = dt;
  a.dt_bias = dt_bias;
  a.A = A;
  a.Bm = B;
  a.Cm = C;
  a.D = D;
  a.z = z;
  a.clamp = dims->dt_max > 0.f;
  a.dt_lo = dims->dt_min;
  a.dt_hi = dims->dt_max;
  a.init = initial_state;
  a.y = y;
  a.final_state = final_state;
  char* ws = static_cast<char*>(workspace);
  a.dtp = has_seq ? reinterpret_cast<float*>(ws + wl.dtp_off) : nullptr;
  a.dAcs = has_seq ? reinterpret_cast<float*>(ws + wl.dacs_off) : nullptr;
  a.states = has_seq ? reinterpret_cast<float*>(ws + wl.states_off) : nullptr;
  a.cb = nullptr;   // set below, once the scan's decomposition is known
  a.cbT = nullptr;
  a.prev16 = has_seq && dims->dtype == SSD_BF16 ? static_cast<void*>(ws + wl.prev16_off) : nullptr;
  a.keep_f32_states = 0;
  a.scan_variant = pick_scan_variant(dims, chunk_size, o);
  a.rows_group = pick_rows_group(o);
  a.heads_per_block = pick_heads_per_block(a.B, a.nc, a.H, a.G, a.scan_variant, o);
  // C B^T blocks for the row blocks and whole chunks to read (the group form forms its own)
  a.cb = has_seq && cb_shared(dims) && a.scan_variant != 3 ? reinterpret_cast<float*>(ws + wl.cb_off) : nullptr;
  a.state_from_start = 0;
  a.passing_reverse = 0;
  a.seg_len = 0;
  a.hin16 = nullptr;
  a.cdec = nullptr;
  a.ev0 = a.ev1 = nullptr;

  if (!has_seq) {
    // no tokens: final_state = initial_state (or zeros); state_passing with zero chunks
    if (ev)
      for (int k = 0; k < 6; ++k)
        if (hipEventRecord(ev[k], stream) != hipSuccess) return SSD_ERR_HIP;
    if (!final_state) return SSD_OK;
    return ssd::launch_state_passing(a, stream) == hipSuccess ? SSD_OK : SSD_ERR_HIP;
  }

  // kernel k is timed by ev[2k] (start) and ev[2k + 1] (stop), recorded by its own dispatch
  auto stage = [&](int k) {
    a.ev0 = ev ? ev[2 * k] : nullptr;
    a.ev1 = ev ? ev[2 * k + 1] : nullptr;
  };
  const StatePath sp = pick_state_path(a.dtype, a.B, a.H, a.G, a.P, a.N, a.Q, a.nc,
                                      !a.keep_f32_states && !a.state_from_start, a.scan_variant, o);
  if (sp.path == 3) {
    // segment states from zero (into the chunk-state region: end states in fp32, then the
    // incoming states in bf16), their exponents in the segments region; state_passing over the
    // segments; the scan adds each segment's incoming state
    ssd::SegArgs sg;
    sg.hs = sp.hs;
    sg.SL = sp.SL;
    sg.nseg = (a.nc + sp.SL - 1) / sp.SL;
    const size_t pnh = (size_t)a.B * sg.nseg * a.H * a.P * a.N;
    sg.E = a.states;
    __bf16* hin16 = reinterpret_cast<__bf16*>(reinterpret_cast<char*>(a.states) + align_up(pnh * sizeof(float)));
    sg.segdec = reinterpret_cast<float*>(ws + wl.segs_off);
    sg.cdec = sg.segdec + align_up((size_t)a.B * a.H * a.nc * sizeof(float)) / sizeof(float);
    stage(0);
    if (ssd::launch_chunk_state_seg(a, sg, stream) != hipSuccess) return SSD_ERR_HIP;
    ssd::FwdArgs cp = a;   // the recurrence over segments: "chunks" of length 1 with the segments' exponents
    cp.nc = sg.nseg;
    cp.Q = 1;
    cp.dAcs = sg.segdec;
    cp.states = sg.E;
    cp.prev16 = hin16;
    cp.keep_f32_states = 0;
    cp.ev0 = ev ? ev[2] : nullptr;
    cp.ev1 = ev ? ev[3] : nullptr;
    if (ssd::launch_state_passing(cp, stream) != hipSuccess) return SSD_ERR_HIP;
    a.seg_len = sp.SL;
    a.hin16 = hin16;
    a.cdec = sg.cdec;
  } else if (sp.path == 2) {
    stage(0);
    if (ssd::launch_chunk_state_seq(a, sp.ps, stream) != hipSuccess) return SSD_ERR_HIP;
    // no state_passing launch: its event pair brackets nothing
    if (ev && (hipEventRecord(ev[2], stream) != hipSuccess || hipEventRecord(ev[3], stream) != hipSuccess))
      return SSD_ERR_HIP;
  } else {
    stage(0);
    if (ssd::launch_chunk_state(a, stream) != hipSuccess) return SSD_ERR_HIP;
    stage(1);
    if (ssd::launch_state_passing(a, stream) != hipSuccess) return SSD_ERR_HIP;
  }
  stage(2);
  if (ssd::launch_chunk_scan(a, stream) != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

// Backward workspace: the forward's regions, the state gradients, per-head dB / dC, per-token
// and per-chunk partials, and (with a gate) the pre-gate output and the gated gradient.
struct BwdLayout {
  size_t dtp, dacs, states, gstates, dBh, dCh, ddir, dSa, dSc, Ub, pA, pbias, pD, ypre, dyg, cb, cbT, prev16, total;
};

// Heads per bwd_dxdb / bwd_dc workgroup (their dB / dC summed on chip, in head order): 1 or,
// for bf16 inputs, 4 -- the option when it is one of those and divides the heads of a group,
// else 4 for bf16 when it divides them and leaves at least 1024 workgroups.
int pick_bwd_heads(const ssd_dims_t* d, int Q, const ssd_launch_opts_t& o) {
  const int hpg = (int)(d->nheads / d->ngroups);
  const bool four = d->dtype == SSD_BF16 && hpg % 4 == 0;
  if (o.bwd_heads > 0) return o.bwd_heads == 4 && four ? 4 : 1;
  const int64_t nc = (d->seqlen + Q - 1) / Q;
  const int64_t units = d->batch * nc * (Q / 64) * d->nheads;
  return four && units / 4 >= 1024 ? 4 : 1;
}

BwdLayout bwd_layout(const ssd_dims_t* d, int Q, bool gate) {
  const int64_t nc = (d->seqlen + Q - 1) / Q;
  const size_t cum = align_up((size_t)d->batch * d->nheads * nc * Q * sizeof(float));
  const size_t st = align_up((size_t)d->batch * nc * d->nheads * d->headdim * d->dstate * sizeof(float));
  const size_t perh = align_up((size_t)d->batch * d->seqlen * d->nheads * d->dstate * sizeof(float));
  const size_t par = align_up((size_t)d->batch * nc * d->nheads * sizeof(float));
  const size_t pd = align_up((size_t)d->batch * nc * (Q / 64) * d->nheads * d->headdim * sizeof(float));
  const size_t act = gate ? align_up((size_t)d->batch * d->seqlen * d->nheads * d->headdim * elem_bytes(d->dtype)) : 0;
  BwdLayout w;
  size_t o = 0;
  w.dtp = o; o += cum;
  w.dacs = o; o += cum;
  w.states = o; o += st;
  w.gstates = o; o += st;
  w.dBh = o; o += perh;
  w.dCh = o; o += perh;
  w.ddir = o; o += cum;
  w.dSa = o; o += cum;
  w.dSc = o; o += cum;
  w.Ub = o; o += cum;
  w.pA = o; o += par;
  w.pbias = o; o += par;
  w.pD = o; o += pd;
  w.ypre = o; o += act;
  w.dyg = o; o += act;
  w.cb = o; o += (gate || d->dtype == SSD_F32) ? cb_bytes(d, Q) : 0;
  w.cbT = o; o += d->dtype == SSD_F32 ? cb_bytes(d, Q) : 0;
  w.prev16 = o; o += prev16_bytes(d, Q);                // (bf16 only: zero bytes for fp32)
  w.total = o;
  return w;
}

ssd_status_t bwd_impl(const ssd_dims_t* dims, const void* x, const void* dt, const float* dt_bias, const float* A,
                      const void* B, const void* C, const float* D, const void* z, int chunk_size,
                      const float* initial_state, const void* dout, const float* dfinal_state, void* dx, void* ddt,
                      float* ddt_bias, float* dA, void* dB, void* dC, float* dD, void* dz, float* dinitial_state,
                      void* workspace, size_t workspace_bytes, hipStream_t stream, const ssd_launch_opts_t* opts,
                      hipEvent_t* ev) {
  const ssd_launch_opts_t& o = opts_or_builtin(opts);
  ssd_status_t st = check_dims(dims, true);
  if (st != SSD_OK) return st;
  if (!chunk_ok(chunk_size)) return SSD_ERR_UNSUPPORTED;
  if (!dt_bias || !A || !ddt_bias || !dA) return SSD_ERR_INVALID_ARG;
  if ((z == nullptr) != (dz == nullptr)) return SSD_ERR_INVALID_ARG;   // dz exactly when gated
  // no tokens (seqlen == 0 or batch == 0): only the per-head gradients (zeros) and dinitial_state
  const bool has_seq = dims->seqlen > 0 && dims->batch > 0;
  const size_t eb = elem_bytes(dims->dtype);
  if (has_seq) {
    if (!x || !dt || !B || !C || !dout || !dx || !ddt || !dB || !dC) return SSD_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(dout, 16)) return SSD_ERR_INVALID_ARG;
    if (!aligned(dt, eb) || !aligned(dx, eb) || !aligned(ddt, eb) || !aligned(dB, eb) || !aligned(dC, eb) ||
        (z && (!aligned(z, eb) || !aligned(dz, eb))) || (D && !aligned(D, 4)))
      return SSD_ERR_INVALID_ARG;
  }
  if (!aligned(dt_bias, 4) || !aligned(A, 4) || !aligned(ddt_bias, 4) || !aligned(dA, 4) || (dD && !aligned(dD, 4)))
    return SSD_ERR_INVALID_ARG;
  if ((initial_state && !aligned(initial_state, 16)) || (dfinal_state && !aligned(dfinal_state, 16)) ||
      (dinitial_state && !aligned(dinitial_state, 16)))
    return SSD_ERR_INVALID_ARG;
  const BwdLayout wl = bwd_layout(dims, chunk_size, z != nullptr);
  if (wl.total > 0 && (!workspace || workspace_bytes < wl.total)) return SSD_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, 16)) return SSD_ERR_INVALID_ARG;
  const bool has_b = dims->batch > 0;   // per-sequence tensors are empty when batch == 0
  const void* ptrs[] = {has_seq ? x : nullptr, has_seq ? dt : nullptr, dt_bias, A, has_seq ? B : nullptr,
                        has_seq ? C : nullptr, D, has_seq ? z : nullptr, has_b ? initial_state : nullptr,
                        has_seq ? dout : nullptr, has_b ? dfinal_state : nullptr, has_seq ? dx : nullptr,
                        has_seq ? ddt : nullptr, ddt_bias, dA, has_seq ? dB : nullptr, has_seq ? dC : nullptr, dD,
                        has_seq ? dz : nullptr, has_b ? dinitial_state : nullptr, wl.total > 0 ? workspace : nullptr};
  for (const void* p : ptrs)
    if (p && !device_ptr_ok(p)) return SSD_ERR_DEVICE_PTR;
  if (ev) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return SSD_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) return SSD_ERR_UNSUPPORTED;
  }

  char* ws = static_cast<char*>(workspace);
  ssd::BwdArgs a;
  ssd::FwdArgs& f = a.f;
  f.B = (int)dims->batch;
  f.L = (int)dims->seqlen;
  f.H = (int)dims->nheads;
  f.P = (int)dims->headdim;
  f.N = (int)dims->dstate;
  f.G = (int)dims->ngroups;
  f.Q = chunk_size;
  f.nc = (int)((dims->seqlen + chunk_size - 1) / chunk_size);
  f.dtype = dims->dtype;
  f.x = x;
  f.dt = dt;
  f.dt_bias = dt_bias;
  f.A = A;
  f.Bm = B;
  f.Cm = C;
  f.D = D;
  f.z = nullptr;                                      // the recomputed output is the pre-gate one
  f.clamp = dims->dt_max > 0.f;
  f.dt_lo = dims->dt_min;
  f.dt_hi = dims->dt_max;
  f.init = initial_state;
  f.y = ws + wl.ypre;
  f.final_state = nullptr;
  f.dtp = reinterpret_cast<float*>(ws + wl.dtp);
  f.dAcs = reinterpret_cast<float*>(ws + wl.dacs);
  f.states = reinterpret_cast<float*>(ws + wl.states);
  // C B^T once per group (when shared): read by the scan for the pre-gate output and, for fp32,
  // by bwd_dc (fp32 B4 L1024 H24: bwd_dc 86.5 -> 69.1 us; for bf16 forming C B^T from the bf16
  // rows in bwd_dc measured as fast as reading the blocks, which then only cost chunk_state)
  f.cb = cb_shared(dims) && (z || dims->dtype == SSD_F32) ? reinterpret_cast<float*>(ws + wl.cb) : nullptr;
  // fp32: the same blocks transposed for bwd_dxdb
  f.cbT = dims->dtype == SSD_F32 ? reinterpret_cast<float*>(ws + wl.cbT) : nullptr;
  // bf16: state_passing also writes the entering states rounded to bf16, which bwd_dc stages
  // (and the gated path's pre-gate chunk_scan reads)
  f.prev16 = dims->dtype == SSD_BF16 ? static_cast<void*>(ws + wl.prev16) : nullptr;
  f.keep_f32_states = 1;                              // bwd_finalize (and fp32 bwd_dc) read the fp32 states
  f.scan_variant = pick_scan_variant(dims, chunk_size, o);
  f.rows_group = pick_rows_group(o);
  f.heads_per_block = pick_heads_per_block(f.B, f.nc, f.H, f.G, f.scan_variant, o);
  if (f.scan_variant == 3 && dims->dtype != SSD_F32) f.cb = nullptr;   // the group form forms its own
  f.state_from_start = 0;
  f.passing_reverse = 0;
  f.seg_len = 0;
  f.hin16 = nullptr;
  f.cdec = nullptr;
  f.ev0 = f.ev1 = nullptr;
  a.dy = z ? static_cast<const void*>(ws + wl.dyg) : dout;
  a.hs_dxdb = pick_bwd_heads(dims, chunk_size, o);
  a.hs_dc = a.hs_dxdb;
  a.gstates = reinterpret_cast<float*>(ws + wl.gstates);
  a.dBh = reinterpret_cast<float*>(ws + wl.dBh);
  a.dCh = reinterpret_cast<float*>(ws + wl.dCh);
  a.ddir = reinterpret_cast<float*>(ws + wl.ddir);
  a.dSa = reinterpret_cast<float*>(ws + wl.dSa);
  a.dSc = reinterpret_cast<float*>(ws + wl.dSc);
  a.Ub = reinterpret_cast<float*>(ws + wl.Ub);
  a.pA = reinterpret_cast<float*>(ws + wl.pA);
  a.pbias = reinterpret_cast<float*>(ws + wl.pbias);
  a.pD = reinterpret_cast<float*>(ws + wl.pD);
  a.dx = dx;
  a.ddt = ddt;
  a.dB = dB;
  a.dC = dC;
  a.ddt_bias = ddt_bias;
  a.dA = dA;
  a.dD = dD;

  // the state gradients, run backwards over the chunks from dL/dfinal_state
  ssd::FwdArgs gp = f;
  gp.states = a.gstates;
  gp.init = dfinal_state;
  gp.final_state = dinitial_state;
  gp.passing_reverse = 1;
  gp.prev16 = nullptr;
  // stage k is timed by ev[2k] (start) and ev[2k + 1] (stop), recorded by the dispatches
  // themselves; stages that launch nothing record both events back to back
  auto timing = [&](ssd::FwdArgs& args, int k) {
    args.ev0 = ev ? ev[2 * k] : nullptr;
    args.ev1 = ev ? ev[2 * k + 1] : nullptr;
  };
  auto empty_stage = [&](int k) {
    return !ev || (hipEventRecord(ev[2 * k], stream) == hipSuccess && hipEventRecord(ev[2 * k + 1], stream) == hipSuccess);
  };
  if (!has_seq) {
    for (int k = 0; k < 10; ++k)
      if (!empty_stage(k)) return SSD_ERR_HIP;
    if (has_b && dinitial_state && ssd::launch_state_passing(gp, stream) != hipSuccess) return SSD_ERR_HIP;
    if (ssd::launch_bwd_reduce(a, stream) != hipSuccess) return SSD_ERR_HIP;   // zero dA, d dt_bias, dD
    return SSD_OK;
  }
  // forward intermediates: dt', its cumsum, the states entering each chunk, and (when shared)
  // the C B^T blocks
  timing(f, 0);
  if (ssd::launch_chunk_state(f, stream) != hipSuccess) return SSD_ERR_HIP;
  timing(f, 1);
  if (ssd::launch_state_passing(f, stream) != hipSuccess) return SSD_ERR_HIP;
  if (z) {
    // pre-gate output, then dy = dout silu(z) and dz = dout y~ silu'(z)
    timing(f, 2);
    if (ssd::launch_chunk_scan(f, stream) != hipSuccess) return SSD_ERR_HIP;
    ssd::GateArgs ga;
    ga.n = dims->batch * dims->seqlen * dims->nheads * dims->headdim;
    ga.dtype = dims->dtype;
    ga.dout = dout;
    ga.z = z;
    ga.ypre = f.y;
    ga.dy = ws + wl.dyg;
    ga.dz = dz;
    ga.ev0 = ev ? ev[6] : nullptr;
    ga.ev1 = ev ? ev[7] : nullptr;
    if (ssd::launch_gate_bwd(ga, stream) != hipSuccess) return SSD_ERR_HIP;
  } else if (!empty_stage(2) || !empty_stage(3)) {
    return SSD_ERR_HIP;
  }
  // per-chunk gradient into the entering state: sum_i exp(dAcs_i) dy_i^T C_i
  ssd::FwdArgs gs = f;
  gs.x = a.dy;
  gs.Bm = C;
  gs.states = a.gstates;
  gs.state_from_start = 1;
  timing(gs, 4);
  if (ssd::launch_chunk_state(gs, stream) != hipSuccess) return SSD_ERR_HIP;
  timing(gp, 5);
  if (ssd::launch_state_passing(gp, stream) != hipSuccess) return SSD_ERR_HIP;
  timing(f, 6);
  if (ssd::launch_bwd_dxdb(a, stream) != hipSuccess) return SSD_ERR_HIP;
  timing(f, 7);
  if (ssd::launch_bwd_dc(a, stream) != hipSuccess) return SSD_ERR_HIP;
  timing(f, 8);
  if (ssd::launch_bwd_finalize(a, stream) != hipSuccess) return SSD_ERR_HIP;
  timing(f, 9);
  if (ssd::launch_bwd_reduce(a, stream) != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

// ssd_step (events: start / stop recorded by the kernel's dispatch, or null)
ssd_status_t step_impl(const ssd_dims_t* dims, float* state, const void* x, const void* dt, const float* dt_bias,
                       const float* A, const void* B, const void* C, const float* D, const void* z, void* y,
                       hipStream_t stream, hipEvent_t* ev) {
  ssd_status_t st = check_dims(dims, false);
  if (st != SSD_OK) return st;
  if (dims->batch == 0) return SSD_OK;
  const size_t eb = elem_bytes(dims->dtype);
  if (!state || !x || !dt || !dt_bias || !A || !B || !C || !y) return SSD_ERR_INVALID_ARG;
  if (!aligned(state, 16) || !aligned(x, eb) || !aligned(dt, eb) || !aligned(B, eb) || !aligned(C, eb) ||
      !aligned(y, eb) || !aligned(dt_bias, 4) || !aligned(A, 4) || (D && !aligned(D, 4)) || (z && !aligned(z, eb)))
    return SSD_ERR_INVALID_ARG;
  const void* ptrs[] = {state, x, dt, dt_bias, A, B, C, D, z, y};
  for (const void* p : ptrs)
    if (p && !device_ptr_ok(p)) return SSD_ERR_DEVICE_PTR;
  if (ev) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return SSD_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) return SSD_ERR_UNSUPPORTED;
  }
  ssd::StepArgs a;
  a.B = (int)dims->batch;
  a.H = (int)dims->nheads;
  a.P = (int)dims->headdim;
  a.N = (int)dims->dstate;
  a.G = (int)dims->ngroups;
  a.dtype = dims->dtype;
  a.state = state;
  a.x = x;
  a.dt = dt;
  a.dt_bias = dt_bias;
  a.A = A;
  a.Bm = B;
  a.Cm = C;
  a.D = D;
  a.z = z;
  a.clamp = dims->dt_max > 0.f;
  a.dt_lo = dims->dt_min;
  a.dt_hi = dims->dt_max;
  a.y = y;
  a.ev0 = ev ? ev[0] : nullptr;
  a.ev1 = ev ? ev[1] : nullptr;
  return ssd::launch_ssd_step(a, stream) == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

// ---------------------------------------------------------------- no-allocation forward
// The workspace of ssd_fwd_noalloc: a fixed device array of the library (each device that runs
// the library holds its own copy until the process ends).  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the device address is
// resolved once per device with hipGetSymbolAddress, with that device current, and kept here.
constexpr size_t kScratchBytes = SSD_FWD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // written once per device, under g_scratch_mu

// Device address of `scratch` on the current device (resolved on the first call there).
ssd_status_t scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSD_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return SSD_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SSD_OK;
}

// Both conv entry points.  `step`: one token per sequence, state updated in place.
ssd_status_t conv_impl(const ssd_dims_t* dims, int K, const void* xbc, const float* weight, const float* bias,
                       const void* state_in, void* state_out, void* x, void* B, void* C, hipStream_t stream,
                       bool step, const ssd_launch_opts_t* opts) {
  ssd_status_t st = check_dims(dims, !step);
  if (st != SSD_OK) return st;
  if (K < 1 || K > 4) return SSD_ERR_UNSUPPORTED;
  if (dims->batch == 0) return SSD_OK;
  const bool has_seq = step || dims->seqlen > 0;
  const size_t eb = elem_bytes(dims->dtype);
  const int64_t dx = dims->nheads * dims->headdim, dbc = dims->ngroups * dims->dstate;
  const int64_t Dc = dx + 2 * dbc;
  if (Dc > (int64_t)1 << 24) return SSD_ERR_UNSUPPORTED;
  // thread count of the prefill launch at its shortest segment (16 tokens) and vector (4 channels)
  if (!step && dims->batch * ((dims->seqlen + 15) / 16 + 1) * (Dc / 4) > ((int64_t)1 << 32) - 256)
    return SSD_ERR_UNSUPPORTED;
  if (has_seq) {
    if (!xbc || !weight || !x || !B || !C) return SSD_ERR_INVALID_ARG;
    if (!aligned(xbc, 16) || !aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(weight, 4) ||
        (bias && !aligned(bias, 4)))
      return SSD_ERR_INVALID_ARG;
  }
  if (step && K > 1 && !state_out) return SSD_ERR_INVALID_ARG;       // decoding needs the state
  if ((state_in && !aligned(state_in, 16)) || (state_out && !aligned(state_out, 16))) return SSD_ERR_INVALID_ARG;
  // the incoming and outgoing states are either the same buffer or disjoint
  if (K > 1 && state_in && state_out && state_in != state_out) {
    const size_t bytes = (size_t)dims->batch * (K - 1) * Dc * eb;
    const char* a = static_cast<const char*>(state_in);
    const char* o = static_cast<const char*>(state_out);
    if (a < o + bytes && o < a + bytes) return SSD_ERR_INVALID_ARG;
  }
  const void* ptrs[] = {has_seq ? xbc : nullptr, has_seq ? weight : nullptr, has_seq ? bias : nullptr,
                        K > 1 ? state_in : nullptr, K > 1 ? state_out : nullptr,
                        has_seq ? x : nullptr, has_seq ? B : nullptr, has_seq ? C : nullptr};
  for (const void* p : ptrs)
    if (p && !device_ptr_ok(p)) return SSD_ERR_DEVICE_PTR;
  if (!has_seq && (K == 1 || !state_out)) return SSD_OK;              // no tokens and no state to write

  ssd::ConvArgs a;
  a.B = (int)dims->batch;
  a.L = step ? 1 : (int)dims->seqlen;
  a.Dc = (int)Dc;
  a.dx = (int)dx;
  a.dbc = (int)dbc;
  a.K = K;
  a.dtype = dims->dtype;
  a.xbc = xbc;
  a.w = weight;
  a.bias = bias;
  a.state_in = state_in;
  a.state_out = state_out;
  a.x = x;
  a.Bo = B;
  a.Co = C;
  a.segment = opts && opts->conv_tokens > 0 ? opts->conv_tokens : 0;
  const hipError_t e = step ? ssd::launch_conv1d_silu_step(a, stream) : ssd::launch_conv1d_silu(a, stream);
  return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // namespace

namespace ssd {
bool shape_supported(int dtype, int P, int N) {
#define SSD_CASE(T, P_, N_) \
  if (dtype == SSD_DTYPE_CODE_##T && P == P_ && N == N_) return true;
  SSD_FOR_EACH_SHAPE(SSD_CASE)
#undef SSD_CASE
  return false;
}
}  // namespace ssd

extern "C" {

size_t ssd_fwd_workspace_size(const ssd_dims_t* dims, int chunk_size) {
  if (check_dims(dims, true) != SSD_OK || !chunk_ok(chunk_size)) return 0;
  return ws_layout(dims, chunk_size).total;
}

ssd_status_t ssd_fwd(const ssd_dims_t* dims, const void* x, const void* dt, const float* dt_bias, const float* A,
                     const void* B, const void* C, const float* D, const void* z, int chunk_size,
                     const float* initial_state, void* y, float* final_state, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  return fwd_impl(dims, x, dt, dt_bias, A, B, C, D, z, chunk_size, initial_state, y, final_state, workspace,
                  workspace_bytes, stream, nullptr, nullptr);
}

ssd_status_t ssd_fwd_ex(const ssd_dims_t* dims, const void* x, const void* dt, const float* dt_bias, const float* A,
                        const void* B, const void* C, const float* D, const void* z, int chunk_size,
                        const float* initial_state, void* y, float* final_state, void* workspace,
                        size_t workspace_bytes, hipStream_t stream, const ssd_launch_opts_t* opts,
                        hipEvent_t* stage_events) {
  return fwd_impl(dims, x, dt, dt_bias, A, B, C, D, z, chunk_size, initial_state, y, final_state, workspace,
                  workspace_bytes, stream, opts, stage_events);
}

ssd_status_t ssd_fwd_noalloc(const ssd_dims_t* dims, const void* x, const void* dt, const float* dt_bias,
                             const float* A, const void* B, const void* C, const float* D, const void* z,
                             int chunk_size, const float* initial_state, void* y, float* final_state,
                             hipStream_t stream) {
  ssd_status_t st = check_dims(dims, true);
  if (st != SSD_OK) return st;
  if (!chunk_ok(chunk_size)) return SSD_ERR_UNSUPPORTED;
  // sizes beyond the fixed scratch are refused before anything else happens
  if (ws_layout(dims, chunk_size).total > kScratchBytes) return SSD_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != SSD_OK) return st;
  return fwd_impl(dims, x, dt, dt_bias, A, B, C, D, z, chunk_size, initial_state, y, final_state, ws, kScratchBytes,
                  stream, nullptr, nullptr, true);
}

ssd_status_t ssd_step(const ssd_dims_t* dims, float* state, const void* x, const void* dt, const float* dt_bias,
                      const float* A, const void* B, const void* C, const float* D, const void* z, void* y,
                      hipStream_t stream) {
  return step_impl(dims, state, x, dt, dt_bias, A, B, C, D, z, y, stream, nullptr);
}

ssd_status_t ssd_step_ex(const ssd_dims_t* dims, float* state, const void* x, const void* dt, const float* dt_bias,
                         const float* A, const void* B, const void* C, const float* D, const void* z, void* y,
                         hipStream_t stream, hipEvent_t* events) {
  return step_impl(dims, state, x, dt, dt_bias, A, B, C, D, z, y, stream, events);
}

int ssd_bwd_heads(const ssd_dims_t* dims, int chunk_size, const ssd_launch_opts_t* opts) {
  if (check_dims(dims, true) != SSD_OK || !chunk_ok(chunk_size)) return 0;
  return pick_bwd_heads(dims, chunk_size, opts_or_builtin(opts));
}

size_t ssd_bwd_workspace_size(const ssd_dims_t* dims, int chunk_size, int with_gate) {
  if (check_dims(dims, true) != SSD_OK || !chunk_ok(chunk_size)) return 0;
  return bwd_layout(dims, chunk_size, with_gate != 0).total;
}

ssd_status_t ssd_bwd(const ssd_dims_t* dims, const void* x, const void* dt, const float* dt_bias, const float* A,
                     const void* B, const void* C, const float* D, const void* z, int chunk_size,
                     const float* initial_state, const void* dout, const float* dfinal_state, void* dx, void* ddt,
                     float* ddt_bias, float* dA, void* dB, void* dC, float* dD, void* dz, float* dinitial_state,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(dims, x, dt, dt_bias, A, B, C, D, z, chunk_size, initial_state, dout, dfinal_state, dx, ddt,
                  ddt_bias, dA, dB, dC, dD, dz, dinitial_state, workspace, workspace_bytes, stream, nullptr, nullptr);
}

ssd_status_t ssd_bwd_ex(const ssd_dims_t* dims, const void* x, const void* dt, const float* dt_bias, const float* A,
                        const void* B, const void* C, const float* D, const void* z, int chunk_size,
                        const float* initial_state, const void* dout, const float* dfinal_state, void* dx,
                        void* ddt, float* ddt_bias, float* dA, void* dB, void* dC, float* dD, void* dz,
                        float* dinitial_state, void* workspace, size_t workspace_bytes, hipStream_t stream,
                        const ssd_launch_opts_t* opts, hipEvent_t* stage_events) {
  return bwd_impl(dims, x, dt, dt_bias, A, B, C, D, z, chunk_size, initial_state, dout, dfinal_state, dx, ddt,
                  ddt_bias, dA, dB, dC, dD, dz, dinitial_state, workspace, workspace_bytes, stream, opts,
                  stage_events);
}

namespace {
ssd_status_t norm_impl(const ssd_dims_t* dims, const void* y, const void* z, const float* weight, float eps,
                       int norm_heads, void* out, hipStream_t stream, hipEvent_t* events) {
  ssd_status_t st = check_dims(dims, true);
  if (st != SSD_OK) return st;
  if (dims->headdim % 8 != 0) return SSD_ERR_UNSUPPORTED;
  if (norm_heads < 1 || norm_heads > dims->nheads || dims->nheads % norm_heads != 0) return SSD_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || eps > 3.0e38f) return SSD_ERR_INVALID_ARG;          // (NaN and inf fail)
  if (norm_heads * dims->headdim > (int64_t)1 << 24) return SSD_ERR_UNSUPPORTED;
  const int64_t tokens = dims->batch * dims->seqlen;
  if (tokens * (dims->nheads / norm_heads) > ((int64_t)1 << 32) - 4) return SSD_ERR_UNSUPPORTED;
  if (tokens == 0) return SSD_OK;
  if (!y || !weight || !out) return SSD_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(out, 16) || (z && !aligned(z, 16)) || !aligned(weight, 16))
    return SSD_ERR_INVALID_ARG;
  // out is y itself or disjoint from y and z
  const size_t bytes = (size_t)tokens * dims->nheads * dims->headdim * elem_bytes(dims->dtype);
  auto overlap = [&](const void* a) {
    const char* p = static_cast<const char*>(a);
    const char* o = static_cast<const char*>(out);
    return p < o + bytes && o < p + bytes;
  };
  if ((out != y && overlap(y)) || (z && overlap(z))) return SSD_ERR_INVALID_ARG;
  for (const void* p : {y, z, static_cast<const void*>(weight), static_cast<const void*>(out)})
    if (p && !device_ptr_ok(p)) return SSD_ERR_DEVICE_PTR;
  if (events) {                                  // (event records cannot be captured)
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return SSD_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) return SSD_ERR_UNSUPPORTED;
  }
  ssd::NormArgs a;
  a.tokens = tokens;
  a.H = (int)dims->nheads;
  a.P = (int)dims->headdim;
  a.norm_heads = norm_heads;
  a.dtype = dims->dtype;
  a.y = y;
  a.z = z;
  a.weight = weight;
  a.out = out;
  a.eps = eps;
  if (events) {
    a.ev0 = events[0];
    a.ev1 = events[1];
  }
  return ssd::launch_gated_rmsnorm(a, stream) == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}
}  // namespace

ssd_status_t ssd_gated_rmsnorm(const ssd_dims_t* dims, const void* y, const void* z, const float* weight, float eps,
                               int norm_heads, void* out, hipStream_t stream) {
  return norm_impl(dims, y, z, weight, eps, norm_heads, out, stream, nullptr);
}

ssd_status_t ssd_gated_rmsnorm_ex(const ssd_dims_t* dims, const void* y, const void* z, const float* weight,
                                  float eps, int norm_heads, void* out, hipStream_t stream, hipEvent_t* events) {
  return norm_impl(dims, y, z, weight, eps, norm_heads, out, stream, events);
}

ssd_status_t ssd_conv1d_silu(const ssd_dims_t* dims, int conv_width, const void* xbc, const float* weight,
                             const float* bias, const void* conv_state_in, void* conv_state_out, void* x, void* B,
                             void* C, hipStream_t stream) {
  return conv_impl(dims, conv_width, xbc, weight, bias, conv_state_in, conv_state_out, x, B, C, stream, false,
                   nullptr);
}

ssd_status_t ssd_conv1d_silu_ex(const ssd_dims_t* dims, int conv_width, const void* xbc, const float* weight,
                                const float* bias, const void* conv_state_in, void* conv_state_out, void* x,
                                void* B, void* C, hipStream_t stream, const ssd_launch_opts_t* opts) {
  return conv_impl(dims, conv_width, xbc, weight, bias, conv_state_in, conv_state_out, x, B, C, stream, false, opts);
}

ssd_status_t ssd_conv1d_silu_step(const ssd_dims_t* dims, int conv_width, void* conv_state, const void* xbc,
                                  const float* weight, const float* bias, void* x, void* B, void* C,
                                  hipStream_t stream) {
  return conv_impl(dims, conv_width, xbc, weight, bias, conv_state, conv_state, x, B, C, stream, true, nullptr);
}

const char* ssd_status_string(ssd_status_t s) {
  switch (s) {
    case SSD_OK: return "success";
    case SSD_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or misaligned pointer)";
    case SSD_ERR_UNSUPPORTED: return "unsupported size, chunk size or dtype";
    case SSD_ERR_DEVICE_PTR: return "pointer is not device memory of the current device";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_HIP: return "HIP runtime error at launch";
    case SSD_ERR_SCRATCH_LIMIT: return "sizes need more workspace than ssd_fwd_noalloc's fixed scratch holds";
  }
  return "unknown status";
}

int ssd_fwd_state_path(const ssd_dims_t* dims, int chunk_size, const ssd_launch_opts_t* opts) {
  if (check_dims(dims, true) != SSD_OK || !chunk_ok(chunk_size) || dims->seqlen == 0 || dims->batch == 0) return 0;
  const int dtype = dims->dtype == SSD_F32 ? ssd::DT_F32 : ssd::DT_BF16;
  const ssd_launch_opts_t& o = opts_or_builtin(opts);
  const int nc = (int)((dims->seqlen + chunk_size - 1) / chunk_size);
  return pick_state_path(dtype, dims->batch, dims->nheads, dims->ngroups, (int)dims->headdim, (int)dims->dstate,
                         chunk_size, nc, true, pick_scan_variant(dims, chunk_size, o), o).path;
}

int ssd_fwd_state_segment_chunks(const ssd_dims_t* dims, int chunk_size, const ssd_launch_opts_t* opts) {
  if (check_dims(dims, true) != SSD_OK || !chunk_ok(chunk_size) || dims->seqlen == 0 || dims->batch == 0) return 0;
  const int dtype = dims->dtype == SSD_F32 ? ssd::DT_F32 : ssd::DT_BF16;
  const ssd_launch_opts_t& o = opts_or_builtin(opts);
  const int nc = (int)((dims->seqlen + chunk_size - 1) / chunk_size);
  const StatePath sp = pick_state_path(dtype, dims->batch, dims->nheads, dims->ngroups, (int)dims->headdim,
                                       (int)dims->dstate, chunk_size, nc, true, pick_scan_variant(dims, chunk_size, o), o);
  return sp.path == 3 ? sp.SL : 0;
}

}  // extern "C"
