// C ABI of the frame-wise GDN forward path: argument checks, workspace
// planning, kernel dispatch on the caller's stream, status strings and the
// optional per-kernel timing record.  See include/gdn.h for the contract.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gdn_status fail(gdn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

constexpr size_t kAlign = 256;
using gdn::kMaxFramesPerLaunch;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  bool gram;                      // Gram pipeline, bf16 or e4m3 I/O (else the single-pass recurrence)
  size_t bh, esz, nb;
  size_t io_bytes, gb_bytes, state_bytes;
  size_t carrier, snap_frame, norm_frame, gfr_frame, bfr_frame;
};

// Shapes already validated.
Plan make_plan(const gdn_desc* d) {
  Plan p;
  p.bh = (size_t)d->B * (size_t)d->H;
  p.esz = d->io_dtype == GDN_FP8_E4M3 ? 1 : d->io_dtype == GDN_BF16 ? 2 : 4;
  p.nb = (size_t)d->D / 16;
  p.io_bytes = p.bh * (size_t)d->T * (size_t)d->S * (size_t)d->D * p.esz;
  p.gb_bytes = p.bh * (size_t)d->T * 4;
  p.state_bytes = p.bh * (size_t)d->D * (size_t)d->D * 4;
  p.carrier = round_up(p.state_bytes);
  p.gram = d->io_dtype != GDN_F32 && !(d->flags & GDN_FLAG_DIRECT);
  // state snapshots: fp32 for fp32 I/O, else bf16
  p.snap_frame = p.bh * (size_t)d->D * (size_t)d->D * (d->io_dtype == GDN_F32 ? 4 : 2);
  // per-frame staging: the single-pass recurrence writes fp32 norm partials,
  // the Gram pipeline writes G_t and B_t (the readout takes norms from the
  // snapshots)
  p.norm_frame = p.gram ? 0 : p.bh * p.nb * 4;
  p.gfr_frame = p.gram ? p.bh * gdn::gram_frame_bytes(d->D) : 0;
  p.bfr_frame = p.gram ? p.bh * gdn::input_frame_bytes(d->D) : 0;
  return p;
}

size_t ws_bytes_for(const Plan& p, size_t frames) {
  return p.carrier + round_up(frames * p.snap_frame) + round_up(frames * p.norm_frame) +
         round_up(frames * p.gfr_frame) + round_up(frames * p.bfr_frame);
}

gdn_status check_desc(const gdn_desc* d) {
  if (!d) return fail(GDN_ERR_NULL, "desc is NULL");
  if (d->abi_version != GDN_ABI_VERSION)
    return fail(GDN_ERR_ABI, "desc.abi_version %d != library ABI %d", d->abi_version, GDN_ABI_VERSION);
  if (d->io_dtype != GDN_F32 && d->io_dtype != GDN_BF16 && d->io_dtype != GDN_FP8_E4M3)
    return fail(GDN_ERR_DTYPE, "io_dtype %d is not GDN_F32, GDN_BF16 or GDN_FP8_E4M3", d->io_dtype);
  if (d->beta_mode != GDN_BETA_ERASE && d->beta_mode != GDN_BETA_WRITE)
    return fail(GDN_ERR_DTYPE, "beta_mode %d is not GDN_BETA_ERASE or GDN_BETA_WRITE", d->beta_mode);
  if (d->flags & ~(GDN_FLAG_TIME_KERNELS | GDN_FLAG_DIRECT | GDN_FLAG_THREE_PASS | GDN_FLAG_ONE_LAUNCH))
    return fail(GDN_ERR_UNSUPPORTED, "unknown flags 0x%x", d->flags);
  if ((d->flags & GDN_FLAG_THREE_PASS) && (d->flags & GDN_FLAG_ONE_LAUNCH))
    return fail(GDN_ERR_UNSUPPORTED, "GDN_FLAG_THREE_PASS and GDN_FLAG_ONE_LAUNCH exclude each other");
  if ((d->flags & GDN_FLAG_DIRECT) && d->io_dtype == GDN_FP8_E4M3)
    return fail(GDN_ERR_UNSUPPORTED, "GDN_FLAG_DIRECT is for bf16 I/O; e4m3 I/O runs the Gram pipeline only");
  if (d->B < 1 || d->H < 1 || d->T < 1 || d->S < 1 || d->D < 1)
    return fail(GDN_ERR_SHAPE, "B=%d H=%d T=%d S=%d D=%d: every size must be >= 1", d->B, d->H, d->T, d->S, d->D);
  if (d->D % 16 != 0 || d->D > 128)
    return fail(GDN_ERR_UNSUPPORTED, "D=%d: supported head dims are 16, 32, ..., 128", d->D);
  const long double per_head = (long double)d->T * d->S * d->D;
  const int esz = d->io_dtype == GDN_F32 ? 4 : d->io_dtype == GDN_BF16 ? 2 : 1;
  if (per_head * esz >= 2147483648.0L)
    return fail(GDN_ERR_SHAPE, "T*S*D*%d = %.0Lf bytes: one head's q, k, v or o must stay below 2 GiB", esz,
                per_head * esz);
  const long double bh = (long double)d->B * d->H;
  if (bh * d->T >= 2147483648.0L || bh * d->D * d->D >= 2147483648.0L * 8)
    return fail(GDN_ERR_SHAPE, "B*H too large for these T and D");
  if (bh * per_head * 4 >= (long double)SIZE_MAX / 4)
    return fail(GDN_ERR_SHAPE, "tensor sizes overflow size_t");
  return GDN_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool misaligned(const void* p, size_t a) { return p && ((uintptr_t)p % a) != 0; }

// ---------------------------------------------------------------------------
// Kernel timing (GDN_FLAG_TIME_KERNELS): every timed kernel is bracketed by two
// events on its own stream; gdn_kernel_times reads them and returns them to a
// pool for reuse.
// ---------------------------------------------------------------------------
struct TimedKernel {
  int slot;
  hipEvent_t ev[2];
};
std::mutex g_time_mu;
std::vector<TimedKernel> g_timed;          // recorded, not read yet
std::vector<hipEvent_t> g_free_events;     // timing events ready for reuse
double g_time_ms[GDN_KERNEL_SLOTS] = {};
int64_t g_time_n[GDN_KERNEL_SLOTS] = {};
// Unread records are capped: past this many, timed calls launch their kernels
// untimed until gdn_kernel_times has read the record.
constexpr size_t kMaxTimed = size_t(1) << 16;

hipError_t take_timing_event(hipEvent_t* e) {
  {
    std::lock_guard<std::mutex> lk(g_time_mu);
    if (!g_free_events.empty()) {
      *e = g_free_events.back();
      g_free_events.pop_back();
      return hipSuccess;
    }
  }
  return hipEventCreate(e);
}

void give_timing_event(hipEvent_t e) {
  std::lock_guard<std::mutex> lk(g_time_mu);
  g_free_events.push_back(e);
}

// Enqueue one kernel (`fn` launches it on `s`), bracketed by timing events when
// `timed`.
template <class Fn>
hipError_t launch_timed(bool timed, int slot, hipStream_t s, Fn&& fn) {
  if (timed) {
    std::lock_guard<std::mutex> lk(g_time_mu);
    if (g_timed.size() >= kMaxTimed) timed = false;
  }
  if (!timed) return fn();
  TimedKernel tk{slot, {nullptr, nullptr}};
  hipError_t e = take_timing_event(&tk.ev[0]);
  if (e != hipSuccess) return e;
  e = take_timing_event(&tk.ev[1]);
  if (e != hipSuccess) { give_timing_event(tk.ev[0]); return e; }
  e = hipEventRecord(tk.ev[0], s);
  if (e == hipSuccess) e = fn();
  if (e == hipSuccess) e = hipEventRecord(tk.ev[1], s);
  if (e != hipSuccess) {
    give_timing_event(tk.ev[0]);
    give_timing_event(tk.ev[1]);
    return e;
  }
  std::lock_guard<std::mutex> lk(g_time_mu);
  g_timed.push_back(tk);
  return hipSuccess;
}

struct Ptrs {
  const void *q, *k, *v;
  const float *gamma, *beta, *state_in;
  void* o;
  float *state_out, *norms;
};

// Largest frame count per launch whose staging fits a workspace of `wb` bytes
// (the minimum-size check guarantees that one frame fits).
size_t frames_per_launch(const Plan& p, int T, size_t wb) {
  size_t frames = std::min<size_t>((size_t)T, (size_t)kMaxFramesPerLaunch);
  if (ws_bytes_for(p, frames) > wb) {
    size_t lo = 1, hi = frames;           // ws_bytes_for(lo) fits, ws_bytes_for(hi) does not
    while (hi - lo > 1) {
      const size_t mid = lo + (hi - lo) / 2;
      (ws_bytes_for(p, mid) <= wb ? lo : hi) = mid;
    }
    frames = lo;
  }
  return frames;
}

// Side stream of the Gram path, one per (thread, device), created on first use
// at default priority and kept for the life of the process, with a small ring
// of events.  An event is recorded again only after every wait on its
// previous record has been enqueued (the enqueue order below guarantees it).
constexpr int kStateSplit = 6;          // state/readout sub-ranges per gram range (at most)
constexpr int kMinSplitFrames = 32;     // frames per sub-range at least
constexpr double kStateGrow = 1.4;      // size ratio of consecutive sub-ranges
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t ev[kStateSplit + 2] = {};
  SideStream() = default;
  SideStream(const SideStream&) = delete;
  SideStream& operator=(const SideStream&) = delete;
  // Released when the owning thread exits.  Work already enqueued is not
  // affected: a stream or event destroyed while in use is freed by the
  // runtime once that work completes.
  ~SideStream() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
    if (stream) (void)hipStreamDestroy(stream);
  }
};

// Sub-range boundaries bnd[0] = 0 < ... < bnd[n] = tc of a gram range, sizes
// growing by kStateGrow.  The state pass of the first sub-range runs alone, so
// it is kept short; the state of sub-range i+1 runs next to the readout of
// sub-range i, which is HBM-bound and takes longer per frame than the state
// pass does, so the later sub-ranges can grow without stalling the readouts.
// Returns n.
int split_frames(int tc, int bnd[kStateSplit + 1]) {
  const int n = std::max(1, std::min(kStateSplit, tc / kMinSplitFrames));
  const double rn = std::pow(kStateGrow, n);
  bnd[0] = 0;
  for (int i = 1; i < n; ++i) {
    const double frac = kStateGrow == 1.0 ? (double)i / n : (std::pow(kStateGrow, i) - 1.0) / (rn - 1.0);
    bnd[i] = std::max(bnd[i - 1] + 1, (int)std::lround(tc * frac));
  }
  bnd[n] = tc;
  return n;
}
thread_local std::vector<std::unique_ptr<SideStream>> t_side;   // by device id

hipError_t side_stream(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((int)t_side.size() <= dev) t_side.resize(dev + 1);
  if (!t_side[dev]) {
    std::unique_ptr<SideStream> ss(new SideStream());
    e = hipStreamCreateWithFlags(&ss->stream, hipStreamNonBlocking);
    for (hipEvent_t& ev : ss->ev)
      if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;   // a partly built side stream is released here
    t_side[dev] = std::move(ss);
  }
  *out = t_side[dev].get();
  return hipSuccess;
}

// Compute units of the current device (0 when the query fails).
int device_cus() {
  static gdn::DeviceOnce once;
  gdn::LaunchInfo li;
  const hipError_t e = once.get([](int dev, gdn::LaunchInfo& info) {
    return hipDeviceGetAttribute(&info.cus, hipDeviceAttributeMultiprocessorCount, dev);
  }, &li);
  return e == hipSuccess ? li.cus : 0;
}

// Short chunk (at most kTailMaxFrames frames, D <= 112, fewer frames than
// CUs, no norms asked for): the gram pass, then the chain and the readout in
// one launch (gdn_step_tail_kernel), two launches instead of three with the
// same bits.  When state_in and state_out overlap, the gram pass first copies
// state_in to the workspace carrier, which the chain then reads.
bool tail_ok(const gdn_desc* d, const Plan& p, const Ptrs& x, size_t F, int cus) {
  return !(d->flags & GDN_FLAG_THREE_PASS) && !x.norms && F >= (size_t)d->T && d->T <= gdn::kTailMaxFrames &&
         d->D <= 112 && cus > 0 && (long long)p.bh * d->T <= cus;
}

gdn_status run_tail(const gdn_desc* d, const Plan& p, const Ptrs& x, float* carrier, void* gfr, void* bfr,
                    int cus, hipStream_t s) {
  const double c = 1.0 / std::sqrt((double)d->D * (double)d->S);
  const bool timed = (d->flags & GDN_FLAG_TIME_KERNELS) != 0;
  const size_t sb = p.state_bytes;
  const bool alias = overlap(x.state_in, sb, x.state_out, sb);
  gdn::GramArgs ga;
  ga.k = x.k; ga.v = x.v; ga.gfr = gfr; ga.bfr = bfr;
  ga.BH = (int)p.bh; ga.T = d->T; ga.S = d->S; ga.t0 = 0; ga.Tc = d->T;
  ga.kscale = (float)c; ga.kscale2 = (float)(c * c);
  ga.fp8 = d->io_dtype == GDN_FP8_E4M3;
  if (alias) { ga.copy_src = x.state_in; ga.copy_dst = carrier; }
  hipError_t e = launch_timed(timed, GDN_KERNEL_GRAM, s, [&] { return gdn::launch_gram(d->D, ga, s); });
  if (e == hipSuccess) {
    gdn::TailArgs ta;
    ta.q = x.q; ta.o = x.o; ta.gfr = gfr; ta.bfr = bfr; ta.gamma = x.gamma; ta.beta = x.beta;
    ta.state_src = alias ? carrier : x.state_in;
    ta.state_dst = x.state_out;
    ta.BH = (int)p.bh; ta.T = d->T; ta.S = d->S; ta.t0 = 0; ta.Tc = d->T;
    // shares of a frame's chunks: about one workgroup per CU, at least one
    // chunk per wave (each share repeats the chain; on the 4-frame short-clip
    // chunk 4 shares measured best, against 1-3 and 7)
    const long long frames = (long long)p.bh * d->T;
    const int nchunk = (d->S + 31) / 32;
    ta.nsplit = (int)std::max<long long>(1, std::min<long long>(cus / frames, nchunk / (long long)p.nb));
    ta.beta_mode = d->beta_mode; ta.fp8 = d->io_dtype == GDN_FP8_E4M3;
    e = launch_timed(timed, GDN_KERNEL_READOUT, s, [&] { return gdn::launch_step_tail(d->D, ta, cus, s); });
  }
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch (short chunk): %s", hipGetErrorString(e));
  return GDN_OK;
}

// Gram path.  Per range of up to kMaxFramesPerLaunch frames: the gram pass
// (all frames in parallel) on the caller's stream; then the serial state pass
// in kStateSplit sub-ranges on the side stream, and the readout of each
// sub-range on the caller's stream as soon as its states exist.  The state
// pass is latency-bound and light on resources, so the state of sub-range
// i+1 runs on the CUs next to the HBM-bound readout of sub-range i.  The state
// crosses sub-ranges and ranges in fp32, so any split gives the same bits.
gdn_status run_gram(const gdn_desc* d, const Plan& p, const Ptrs& x, void* workspace, size_t wb,
                    hipStream_t s, bool side_ok = true) {
  const size_t F = frames_per_launch(p, d->T, wb);
  unsigned char* ws = (unsigned char*)workspace;
  size_t off = 0;
  auto carve = [&](size_t bytes) { void* r = ws + off; off += round_up(bytes); return r; };
  float* carrier = (float*)carve(p.carrier);
  void* snap = carve(F * p.snap_frame);
  carve(0);
  void* gfr = carve(F * p.gfr_frame);
  void* bfr = carve(F * p.bfr_frame);
  const int cus = device_cus();
  if (tail_ok(d, p, x, F, cus)) return run_tail(d, p, x, carrier, gfr, bfr, cus, s);

  // The state travels between launches through state_out when the caller gave
  // one (in-place per workgroup tile), else through the workspace carrier.
  float* hand = x.state_out ? x.state_out : carrier;
  const double c = 1.0 / std::sqrt((double)d->D * (double)d->S);
  const bool timed = (d->flags & GDN_FLAG_TIME_KERNELS) != 0;
  SideStream* ss = nullptr;
  hipError_t e = hipSuccess;
  int failed_t0 = 0;

  for (int t0 = 0; t0 < d->T && e == hipSuccess; t0 += (int)F) {
    failed_t0 = t0;
    const int tc = (int)std::min<size_t>(F, (size_t)(d->T - t0));
    int bnd[kStateSplit + 1];
    const int nsub = side_ok ? split_frames(tc, bnd) : (bnd[0] = 0, bnd[1] = tc, 1);
    gdn::GramArgs ga;
    ga.k = x.k; ga.v = x.v; ga.gfr = gfr; ga.bfr = bfr;
    ga.BH = (int)p.bh; ga.T = d->T; ga.S = d->S; ga.t0 = t0; ga.Tc = tc;
    ga.kscale = (float)c; ga.kscale2 = (float)(c * c);
    ga.fp8 = d->io_dtype == GDN_FP8_E4M3;
    e = launch_timed(timed, GDN_KERNEL_GRAM, s, [&] { return gdn::launch_gram(d->D, ga, s); });
    hipStream_t st = s;
    if (e == hipSuccess && nsub > 1) {
      e = side_stream(&ss);
      if (e == hipSuccess) {
        st = ss->stream;
        e = hipEventRecord(ss->ev[0], s);
        if (e == hipSuccess) e = hipStreamWaitEvent(st, ss->ev[0], 0);
      }
    }
    // state sub-ranges (side stream), then their readouts (caller's stream)
    for (int i = 0; i < nsub && e == hipSuccess; ++i) {
      const int f0 = bnd[i], f1 = bnd[i + 1];
      gdn::StateArgs sa;
      sa.gfr = gfr; sa.bfr = bfr; sa.gamma = x.gamma; sa.beta = x.beta;
      sa.state_src = (t0 == 0 && i == 0) ? x.state_in : hand;
      sa.state_dst = (t0 + tc >= d->T && i == nsub - 1) ? x.state_out : hand;
      sa.snap = snap;
      sa.BH = (int)p.bh; sa.T = d->T; sa.t0 = t0 + f0; sa.Tc = f1 - f0;
      sa.Fs = tc; sa.f0 = f0; sa.beta_mode = d->beta_mode;
      sa.snap_Fs = tc; sa.snap_f0 = f0;
      e = launch_timed(timed, GDN_KERNEL_STATE, st, [&] { return gdn::launch_state(d->D, sa, st); });
      if (e == hipSuccess && st != s) e = hipEventRecord(ss->ev[1 + i], st);
    }
    for (int i = 0; i < nsub && e == hipSuccess; ++i) {
      const int f0 = bnd[i], f1 = bnd[i + 1];
      if (st != s) e = hipStreamWaitEvent(s, ss->ev[1 + i], 0);
      gdn::ReadoutArgs ro;
      ro.q = x.q; ro.o = x.o; ro.snap = snap; ro.norms = x.norms; ro.norm_part = nullptr;
      ro.BH = (int)p.bh; ro.T = d->T; ro.S = d->S; ro.t0 = t0 + f0; ro.Tc = f1 - f0;
      ro.Fs = tc; ro.f0 = f0; ro.fp8 = d->io_dtype == GDN_FP8_E4M3;
      if (e == hipSuccess)
        e = launch_timed(timed, GDN_KERNEL_READOUT, s, [&] { return gdn::launch_readout(d->D, true, ro, s); });
    }
  }
  if (e != hipSuccess) {
    // keep the caller's stream ordered after anything already on the side stream
    if (ss) {
      const int last = kStateSplit + 1;
      if (hipEventRecord(ss->ev[last], ss->stream) == hipSuccess) (void)hipStreamWaitEvent(s, ss->ev[last], 0);
    }
    return fail(GDN_ERR_HIP, "kernel launch (frames from %d): %s", failed_t0, hipGetErrorString(e));
  }
  return GDN_OK;
}

gdn_status run_direct(const gdn_desc* d, const Plan& p, const Ptrs& x, void* workspace, size_t wb,
                      hipStream_t s) {
  const size_t frames = frames_per_launch(p, d->T, wb);
  unsigned char* ws = (unsigned char*)workspace;
  size_t off = 0;
  auto carve = [&](size_t bytes) { void* r = ws + off; off += round_up(bytes); return r; };
  float* carrier = (float*)carve(p.carrier);
  void* snap = carve(frames * p.snap_frame);
  float* norm_part = (float*)carve(frames * p.norm_frame);

  // The state travels between launches through state_out when the caller gave
  // one (in-place per workgroup tile), else through the workspace carrier.
  float* hand = x.state_out ? x.state_out : carrier;
  const double c = 1.0 / std::sqrt((double)d->D * (double)d->S);
  const bool timed = (d->flags & GDN_FLAG_TIME_KERNELS) != 0;
  const bool bf16 = p.esz == 2;

  for (int t0 = 0; t0 < d->T; t0 += (int)frames) {
    const int tc = (int)std::min<size_t>(frames, (size_t)(d->T - t0));
    const bool last = t0 + tc >= d->T;
    gdn::RecurArgs ra;
    ra.k = x.k; ra.v = x.v; ra.gamma = x.gamma; ra.beta = x.beta;
    ra.state_src = (t0 == 0) ? x.state_in : hand;
    ra.state_dst = last ? x.state_out : hand;
    ra.snap = snap;
    ra.norm_part = x.norms ? norm_part : nullptr;
    ra.units = (int)(p.bh * p.nb);
    ra.T = d->T; ra.S = d->S; ra.t0 = t0; ra.Tc = tc;
    ra.beta_mode = d->beta_mode;
    ra.kscale = (float)c;
    gdn::ReadoutArgs ro;
    ro.q = x.q; ro.o = x.o; ro.snap = snap; ro.norms = x.norms; ro.norm_part = ra.norm_part;
    ro.BH = (int)p.bh; ro.T = d->T; ro.S = d->S; ro.t0 = t0; ro.Tc = tc;
    ro.Fs = tc; ro.f0 = 0; ro.fp8 = 0;
    hipError_t e = launch_timed(timed, GDN_KERNEL_RECURRENCE, s,
                                [&] { return gdn::launch_recurrence(d->D, bf16, ra, s); });
    if (e == hipSuccess)
      e = launch_timed(timed, GDN_KERNEL_READOUT, s, [&] { return gdn::launch_readout(d->D, bf16, ro, s); });
    if (e != hipSuccess)
      return fail(GDN_ERR_HIP, "kernel launch (frames %d..%d): %s", t0, t0 + tc - 1, hipGetErrorString(e));
  }
  return GDN_OK;
}

// ---------------------------------------------------------------------------
// One-launch forward (gdn_fused.hip).  Heads are dealt to the XCDs (head h on
// XCD h mod NX); two workgroups per CU; each XCD needs at least as many stream
// workgroups as chain workgroups.  Ring sizes follow from how many frame
// blocks the XCD's stream workgroups keep in flight: the readout lag L covers
// them (so that a readout rarely waits for its state), the gram ring a few
// frames more (so that a finished gram item rarely waits for its slot).
// ---------------------------------------------------------------------------
struct FusedPlan {
  bool ok = false;
  int nx = 0, grid = 0, RG = 0, RM = 0, L = 0, balance = 0;
  size_t ctl = 0, gring = 0, mring = 0, total = 0;
};

// Work below which the one-launch form is not the default: its fixed cost
// (a cooperative launch of every workgroup, the clear of the control block,
// the serial chain filling and draining the pipeline, about 35-45 us) only
// pays off on long sequences; on a 4-frame streaming chunk or a tiny call the
// three launches finish first.  With e4m3 I/O the frames are half the bytes
// and the serial chain, not the memory traffic, sets the pace, so the one
// launch needs longer calls to win (measured on MI355X, one launch vs three:
// 720p bf16 2.88 vs 3.39 ms; short clip bf16 146 vs 166 us, e4m3 134 vs
// 124 us; 720p e4m3 2.07 vs 2.30 ms; 4-frame chunk 50 vs 22 us).
// GDN_FLAG_ONE_LAUNCH asks for it whatever the size.
constexpr double kOneLaunchMinElems = 67108864.0;      // B*H*T*S*D, bf16 I/O
constexpr double kOneLaunchMinElemsFp8 = 268435456.0;  // e4m3 I/O

FusedPlan make_fused_plan(const gdn_desc* d) {
  FusedPlan f;
  if (d->io_dtype == GDN_F32 || (d->flags & (GDN_FLAG_DIRECT | GDN_FLAG_THREE_PASS))) return f;
  if (!(d->flags & GDN_FLAG_ONE_LAUNCH) &&
      (double)d->B * d->H * d->T * d->S * d->D <
          (d->io_dtype == GDN_BF16 ? kOneLaunchMinElems : kOneLaunchMinElemsFp8))
    return f;
  static gdn::DeviceOnce once;
  gdn::LaunchInfo li;
  const hipError_t e = once.get([](int dev, gdn::LaunchInfo& info) {
    hipError_t r = hipDeviceGetAttribute(&info.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (r == hipSuccess) r = hipDeviceGetAttribute(&info.slots, hipDeviceAttributeNumberOfXccs, dev);
    int coop = 0;
    if (r == hipSuccess) r = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
    if (r == hipSuccess && !coop) info.slots = 0;
    return r;
  }, &li);
  if (e != hipSuccess || li.slots < 1 || li.slots > 16 || li.cus < 2 * li.slots || li.cus % li.slots != 0) return f;
  const int nx = li.slots, per_x = 2 * li.cus / nx;                // two workgroups per CU
  const long long bh = (long long)d->B * d->H;
  const int cw = (d->D / 16 + gdn::kFusedWaves - 1) / gdn::kFusedWaves;   // chain workgroups per head
  const int nh = (int)((bh + nx - 1) / nx);                  // heads on the fullest XCD
  if (nh * cw > per_x / 2) return f;
  // The readouts of the extra head of XCD x < rem run on XCD x + rem (the
  // kernel's head placement); per XCD: ng heads with gram items and chain,
  // nr readout heads, per_x - ng cw stream workgroups.  fly: the frame blocks
  // the stream workgroups of the busiest XCD keep in flight.
  f.balance = 1;
  const int rem = (int)(bh % nx);
  int fly = 1;
  for (int x = 0; x < nx; ++x) {
    const int ng = x < bh ? (int)((bh - x + nx - 1) / nx) : 0;
    const int nr = ng - (x < rem && x + rem < nx ? 1 : 0) + (x >= rem && x < 2 * rem ? 1 : 0);
    if (ng + nr == 0) continue;
    const int ns = per_x - ng * cw;
    fly = std::max(fly, (ns + ng + nr - 1) / (ng + nr));
  }
  f.nx = nx;
  f.grid = 2 * li.cus;
  f.RM = std::min(gdn::kFusedMaxRM, 8);
  f.RG = std::min(gdn::kFusedMaxRG, std::max(10, fly + 6 - f.RM + 3));
  f.L = std::min(fly + 6, f.RG + f.RM - 2);                 // progress needs 4 <= L <= RG + RM - 2
  f.ctl = round_up(gdn::fused_ctl_bytes((int)bh));
  f.gring = round_up((size_t)bh * f.RG * gdn::fused_slot_bytes(d->D));
  f.mring = round_up((size_t)bh * f.RM * (size_t)d->D * d->D * 2);
  f.total = f.ctl + f.gring + f.mring;
  f.ok = true;
  return f;
}

gdn_status run_fused(const gdn_desc* d, const FusedPlan& f, const Ptrs& x, void* workspace, hipStream_t s) {
  unsigned char* ws = (unsigned char*)workspace;
  gdn::FusedArgs fa;
  fa.q = x.q; fa.k = x.k; fa.v = x.v; fa.o = x.o;
  fa.gamma = x.gamma; fa.beta = x.beta; fa.state_in = x.state_in; fa.state_out = x.state_out; fa.norms = x.norms;
  fa.ctl = ws;
  fa.gring = ws + f.ctl;
  fa.mring = ws + f.ctl + f.gring;
  fa.BH = d->B * d->H; fa.T = d->T; fa.S = d->S;
  fa.NX = f.nx; fa.RG = f.RG; fa.RM = f.RM; fa.L = f.L; fa.grid = f.grid; fa.balance = f.balance;
  const double c = 1.0 / std::sqrt((double)d->D * (double)d->S);
  fa.kscale = (float)c; fa.kscale2 = (float)(c * c);
  const bool timed = (d->flags & GDN_FLAG_TIME_KERNELS) != 0;
  const hipError_t e = launch_timed(timed, GDN_KERNEL_FUSED, s, [&] {
    return gdn::launch_fused(d->D, fa, d->io_dtype == GDN_FP8_E4M3, d->beta_mode == GDN_BETA_ERASE, s);
  });
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "one-launch forward: %s", hipGetErrorString(e));
  return GDN_OK;
}

gdn_status run(const gdn_desc* d, const void* q, const void* k, const void* v, const float* gamma,
               const float* beta, const float* state_in, void* o, float* state_out, float* norms,
               void* workspace, size_t workspace_bytes, void* stream, int is_step, bool side_ok = true) {
  gdn_status st = gdn_check_args(d, q, k, v, gamma, beta, state_in, o, state_out, norms, workspace,
                                 workspace_bytes, is_step);
  if (st != GDN_OK) return st;
  const Plan p = make_plan(d);
  const Ptrs x{q, k, v, gamma, beta, state_in, o, state_out, norms};
  hipStream_t s = (hipStream_t)stream;
  if (p.gram) {
    const FusedPlan f = make_fused_plan(d);
    if (f.ok && workspace_bytes >= f.total) return run_fused(d, f, x, workspace, s);
    return run_gram(d, p, x, workspace, workspace_bytes, s, side_ok);
  }
  return run_direct(d, p, x, workspace, workspace_bytes, s);
}

// ---------------------------------------------------------------------------
// Backward.  Workspace, per head and frame (bf16 blocks unless noted): the
// forward replay's G_t and B_t, the snapshots of M_{t-1} (T + 1 slots, slot 0
// the initial state), C_t = ReLU(Q_t)^T dO_t, the snapshots of Lambda_t, the
// adjoint pass's fp32 partial sums and an fp32 carrier.
// ---------------------------------------------------------------------------
struct BackwardPlan {
  size_t bh, gfb, bfb, sfb, pfb, io_bytes, gb_bytes, state_bytes;
  size_t gfr, bfr, cfr, msnap, lsnap, part, carrier, total;
};

// Layout of the saved buffer of a training forward: G_t and B_t of every
// frame (the gram pass's staging layout), bf16 state snapshots in T+1 slots
// (slot 0 the initial state, slot t+1 the state after frame t), and an fp32
// state carrier.
struct SavedPlan {
  size_t gfr, bfr, msnap, carrier, total;
};

SavedPlan make_saved_plan(const gdn_desc* d) {
  SavedPlan p;
  const size_t T = (size_t)d->T, D = (size_t)d->D, bh = (size_t)d->B * (size_t)d->H;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t r = off; off += round_up(bytes); return r; };
  p.gfr = take(bh * T * gdn::gram_frame_bytes(d->D));
  p.bfr = take(bh * T * gdn::input_frame_bytes(d->D));
  p.msnap = take(bh * (T + 1) * D * D * 2);
  p.carrier = take(bh * D * D * 4);
  p.total = off;
  return p;
}

// Workspace of the backward.  With a saved forward (`saved`), G_t, B_t and the
// state snapshots come from it and the workspace holds the rest.
BackwardPlan make_backward_plan(const gdn_desc* d, bool saved = false) {
  BackwardPlan b;
  const size_t T = (size_t)d->T, D = (size_t)d->D, nb = D / 16;
  b.bh = (size_t)d->B * (size_t)d->H;
  b.gfb = gdn::gram_frame_bytes(d->D);
  b.bfb = gdn::input_frame_bytes(d->D);
  b.sfb = D * D * 2;
  b.pfb = nb * nb * 16;
  b.io_bytes = b.bh * T * (size_t)d->S * D * 2;
  b.gb_bytes = b.bh * T * 4;
  b.state_bytes = b.bh * D * D * 4;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t r = off; off += round_up(bytes); return r; };
  b.gfr = saved ? 0 : take(b.bh * T * b.gfb);
  b.bfr = saved ? 0 : take(b.bh * T * b.bfb);
  b.cfr = take(b.bh * T * b.bfb);
  b.msnap = saved ? 0 : take(b.bh * (T + 1) * b.sfb);
  b.lsnap = take(b.bh * T * b.sfb);
  b.part = take(b.bh * T * b.pfb);
  b.carrier = take(b.state_bytes);         // fp32 state / adjoint between sub-range launches
  b.total = off;
  return b;
}

gdn_status check_backward(const gdn_desc* d, const void* q, const void* k, const void* v, const float* gamma,
                          const float* beta, const float* state_in, const void* d_out, const float* d_state_out,
                          const void* dq, const void* dk, const void* dv, const float* d_gamma,
                          const float* d_beta, const float* d_state_in, const void* workspace,
                          size_t workspace_bytes, const void* saved = nullptr, size_t saved_bytes = 0,
                          bool saved_mode = false) {
  g_last_error.clear();
  gdn_status st = check_desc(d);
  if (st != GDN_OK) return st;
  if (d->io_dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "gdn_frame_backward takes bf16 I/O only");
  if (d->flags & GDN_FLAG_DIRECT) return fail(GDN_ERR_UNSUPPORTED, "gdn_frame_backward has no single-pass form");
  if (d->T > kMaxFramesPerLaunch)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_frame_backward takes at most %d frames per call", kMaxFramesPerLaunch);
  if (!q || !k || !v || !d_out) return fail(GDN_ERR_NULL, "q, k, v and d_out are required");
  if (!gamma || !beta) return fail(GDN_ERR_NULL, "gamma and beta are required");
  if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is required (gdn_backward_workspace_size)");
  const BackwardPlan b = make_backward_plan(d, saved_mode);
  if (workspace_bytes < b.total)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes < required %zu", workspace_bytes, b.total);
  if (saved_mode) {
    if (!saved) return fail(GDN_ERR_NULL, "saved is required (the buffer of gdn_frame_forward_train)");
    const size_t need = make_saved_plan(d).total;
    if (saved_bytes < need)
      return fail(GDN_ERR_WORKSPACE, "saved buffer of %zu bytes < required %zu", saved_bytes, need);
    if (misaligned(saved, kAlign)) return fail(GDN_ERR_ALIGN, "saved must be 256-byte aligned");
  }
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(d_out, 16) || misaligned(dq, 16) ||
      misaligned(dk, 16) || misaligned(dv, 16))
    return fail(GDN_ERR_ALIGN, "q, k, v, d_out, dq, dk and dv must be 16-byte aligned");
  if (misaligned(gamma, 4) || misaligned(beta, 4) || misaligned(state_in, 4) || misaligned(d_state_out, 4) ||
      misaligned(d_gamma, 4) || misaligned(d_beta, 4) || misaligned(d_state_in, 4))
    return fail(GDN_ERR_ALIGN, "gamma, beta, states and their gradients must be 4-byte aligned");
  if (misaligned(workspace, kAlign)) return fail(GDN_ERR_ALIGN, "workspace must be 256-byte aligned");
  struct Buf { const void* p; size_t n; const char* name; };
  const Buf ins[] = {{q, b.io_bytes, "q"}, {k, b.io_bytes, "k"}, {v, b.io_bytes, "v"},
                     {d_out, b.io_bytes, "d_out"}, {gamma, b.gb_bytes, "gamma"}, {beta, b.gb_bytes, "beta"},
                     {state_in, b.state_bytes, "state_in"}, {d_state_out, b.state_bytes, "d_state_out"},
                     {saved, saved_bytes, "saved"}};
  const Buf outs[] = {{dq, b.io_bytes, "dq"}, {dk, b.io_bytes, "dk"}, {dv, b.io_bytes, "dv"},
                      {d_gamma, b.gb_bytes, "d_gamma"}, {d_beta, b.gb_bytes, "d_beta"},
                      {d_state_in, b.state_bytes, "d_state_in"}, {workspace, workspace_bytes, "workspace"}};
  for (const Buf& x : outs) {
    if (!x.p) continue;
    for (const Buf& y : ins)
      if (overlap(x.p, x.n, y.p, y.n)) return fail(GDN_ERR_ALIAS, "%s overlaps %s", x.name, y.name);
    for (const Buf& y : outs)
      if (&y != &x && y.p && overlap(x.p, x.n, y.p, y.n))
        return fail(GDN_ERR_ALIAS, "%s overlaps %s", x.name, y.name);
  }
  return GDN_OK;
}

gdn_status check_tconv(const gdn_tconv_desc* d, const void* x, const float* w, const float* bias,
                       const void* cache_in, const void* y, const void* cache_out) {
  g_last_error.clear();
  if (!d) return fail(GDN_ERR_NULL, "desc is NULL");
  if (d->abi_version != GDN_ABI_VERSION)
    return fail(GDN_ERR_ABI, "desc.abi_version %d != library ABI %d", d->abi_version, GDN_ABI_VERSION);
  if (d->io_dtype != GDN_F32 && d->io_dtype != GDN_BF16)
    return fail(GDN_ERR_DTYPE, "io_dtype %d: the temporal convolution takes GDN_BF16 or GDN_F32", d->io_dtype);
  if (d->flags & ~GDN_FLAG_TIME_KERNELS) return fail(GDN_ERR_UNSUPPORTED, "unknown flags 0x%x", d->flags);
  if (d->B < 1 || d->T < 1 || d->S < 1 || d->C < 1 || d->chunk < 1)
    return fail(GDN_ERR_SHAPE, "B=%d T=%d S=%d C=%d chunk=%d: every size must be >= 1", d->B, d->T, d->S, d->C,
                d->chunk);
  if (d->C % 8 != 0) return fail(GDN_ERR_UNSUPPORTED, "C=%d: channels must be a multiple of 8", d->C);
  if (d->B > 65535) return fail(GDN_ERR_SHAPE, "B=%d: at most 65535", d->B);
  const long double elems = (long double)d->B * d->T * d->S * d->C;
  if (elems * 4 >= (long double)SIZE_MAX / 4 || (long double)d->S * d->C >= 2147483648.0L * 4)
    return fail(GDN_ERR_SHAPE, "tensor sizes overflow");
  if (!x || !w || !y) return fail(GDN_ERR_NULL, "x, w and y are required");
  if (misaligned(x, 16) || misaligned(y, 16) || misaligned(cache_in, 16) || misaligned(cache_out, 16))
    return fail(GDN_ERR_ALIGN, "x, y and the caches must be 16-byte aligned");
  if (misaligned(w, 4) || misaligned(bias, 4)) return fail(GDN_ERR_ALIGN, "w and bias must be 4-byte aligned");
  const size_t esz = d->io_dtype == GDN_F32 ? 4 : 2;
  const size_t xb = (size_t)d->B * d->T * d->S * d->C * esz, cb = (size_t)d->B * d->S * d->C * esz;
  const size_t wb = (size_t)3 * d->C * 4, bb = (size_t)d->C * 4;
  if (overlap(y, xb, x, xb) || overlap(y, xb, w, wb) || overlap(y, xb, bias, bb) || overlap(y, xb, cache_in, cb))
    return fail(GDN_ERR_ALIAS, "y overlaps an input");
  if (overlap(cache_out, cb, x, xb) || overlap(cache_out, cb, y, xb) || overlap(cache_out, cb, w, wb) ||
      overlap(cache_out, cb, bias, bb))
    return fail(GDN_ERR_ALIAS, "cache_out overlaps x, y, w or bias");
  if (cache_out && cache_in && cache_out != cache_in && overlap(cache_out, cb, cache_in, cb))
    return fail(GDN_ERR_ALIAS, "cache_out partially overlaps cache_in");
  return GDN_OK;
}

gdn_status check_attn_desc(const gdn_attn_desc* d) {
  g_last_error.clear();
  if (!d) return fail(GDN_ERR_NULL, "desc is NULL");
  if (d->abi_version != GDN_ABI_VERSION)
    return fail(GDN_ERR_ABI, "desc.abi_version %d != library ABI %d", d->abi_version, GDN_ABI_VERSION);
  if (d->io_dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "io_dtype %d: the attention takes GDN_BF16", d->io_dtype);
  if (d->flags & ~GDN_FLAG_TIME_KERNELS) return fail(GDN_ERR_UNSUPPORTED, "unknown flags 0x%x", d->flags);
  if (d->B < 1 || d->H < 1 || d->Tq < 1 || d->Tk < 1 || d->S < 1 || d->D < 1 || d->chunk < 1)
    return fail(GDN_ERR_SHAPE, "B=%d H=%d Tq=%d Tk=%d S=%d D=%d chunk=%d: every size must be >= 1", d->B, d->H,
                d->Tq, d->Tk, d->S, d->D, d->chunk);
  if (d->Tq > d->Tk) return fail(GDN_ERR_SHAPE, "Tq=%d > Tk=%d: the queries are the last Tq key frames", d->Tq, d->Tk);
  if (d->D % 16 != 0 || d->D > 128)
    return fail(GDN_ERR_UNSUPPORTED, "D=%d: supported head dims are 16, 32, ..., 128", d->D);
  if (!std::isfinite(d->scale) || d->scale < 0.f)
    return fail(GDN_ERR_SHAPE, "scale must be finite and >= 0 (0 selects 1/sqrt(D))");
  const long double nk = (long double)d->Tk * d->S, bh = (long double)d->B * d->H;
  if (nk * d->D * 2 >= 2147483648.0L || bh * ((long double)d->Tq * d->S / 128 + 1) >= 2147483648.0L)
    return fail(GDN_ERR_SHAPE, "too many tokens per head: Tk*S*D*2 bytes must stay below 2 GiB");
  if (bh * nk * d->D * 2 >= (long double)SIZE_MAX / 4) return fail(GDN_ERR_SHAPE, "tensor sizes overflow");
  return GDN_OK;
}

gdn_status check_attn(const gdn_attn_desc* d, const void* q, const void* k, const void* v, const void* o,
                      const void* workspace, size_t workspace_bytes) {
  const gdn_status st = check_attn_desc(d);
  if (st != GDN_OK) return st;
  if (!q || !k || !v || !o) return fail(GDN_ERR_NULL, "q, k, v and o are required");
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16))
    return fail(GDN_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  const size_t qb = (size_t)d->B * d->H * d->Tq * d->S * d->D * 2, kb = (size_t)d->B * d->H * d->Tk * d->S * d->D * 2;
  if (overlap(o, qb, q, qb) || overlap(o, qb, k, kb) || overlap(o, qb, v, kb))
    return fail(GDN_ERR_ALIAS, "o overlaps q, k or v");
  if (workspace && workspace_bytes) {
    if (misaligned(workspace, kAlign)) return fail(GDN_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (overlap(workspace, workspace_bytes, q, qb) || overlap(workspace, workspace_bytes, k, kb) ||
        overlap(workspace, workspace_bytes, v, kb) || overlap(workspace, workspace_bytes, o, qb))
      return fail(GDN_ERR_ALIAS, "workspace overlaps q, k, v or o");
  }
  return GDN_OK;
}

// Key-split parts for an attention launch on the current device (1 if the
// device cannot be queried).
int attn_parts(const gdn_attn_desc* d) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 1;
  return gdn::attn_split_parts(d->D, d->B * d->H, d->Tq, d->Tk, d->S, d->chunk, cus);
}

// Training forward after its argument check: the forward of run_gram with
// every frame in one gram range, G_t, B_t and the state snapshots kept in the
// caller's saved buffer (snapshot slot t+1 holds M_t, slot 0 the initial
// state) for gdn_frame_backward_saved.
gdn_status run_train(const gdn_desc* d, const Ptrs& x, unsigned char* sv, hipStream_t s) {
  const SavedPlan sp = make_saved_plan(d);
  const int BH = d->B * d->H, T = d->T, D = d->D;
  void* gfr = sv + sp.gfr;
  void* bfr = sv + sp.bfr;
  void* msnap = sv + sp.msnap;
  float* carrier = (float*)(sv + sp.carrier);
  const double c = 1.0 / std::sqrt((double)D * (double)d->S);
  const bool timed = (d->flags & GDN_FLAG_TIME_KERNELS) != 0;
  hipError_t e = gdn::launch_state_snapshot(x.state_in, msnap, BH, D, (size_t)(T + 1) * D * D * 2, s);
  gdn::GramArgs ga;
  ga.k = x.k; ga.v = x.v; ga.gfr = gfr; ga.bfr = bfr;
  ga.BH = BH; ga.T = T; ga.S = d->S; ga.t0 = 0; ga.Tc = T;
  ga.kscale = (float)c; ga.kscale2 = (float)(c * c); ga.fp8 = 0;
  if (e == hipSuccess) e = launch_timed(timed, GDN_KERNEL_GRAM, s, [&] { return gdn::launch_gram(D, ga, s); });
  int bnd[kStateSplit + 1];
  const int nsub = split_frames(T, bnd);
  SideStream* ss = nullptr;
  hipStream_t st = s;
  if (e == hipSuccess && nsub > 1) {
    e = side_stream(&ss);
    if (e == hipSuccess) {
      st = ss->stream;
      e = hipEventRecord(ss->ev[0], s);
      if (e == hipSuccess) e = hipStreamWaitEvent(st, ss->ev[0], 0);
    }
  }
  for (int i = 0; i < nsub && e == hipSuccess; ++i) {
    gdn::StateArgs sa;
    sa.gfr = gfr; sa.bfr = bfr; sa.gamma = x.gamma; sa.beta = x.beta;
    sa.state_src = i == 0 ? x.state_in : carrier;
    sa.state_dst = i == nsub - 1 ? x.state_out : carrier;
    sa.snap = msnap;
    sa.BH = BH; sa.T = T; sa.t0 = bnd[i]; sa.Tc = bnd[i + 1] - bnd[i]; sa.Fs = T; sa.f0 = bnd[i];
    sa.beta_mode = d->beta_mode;
    sa.snap_Fs = T + 1; sa.snap_f0 = 1 + bnd[i];
    e = launch_timed(timed, GDN_KERNEL_STATE, st, [&] { return gdn::launch_state(D, sa, st); });
    if (e == hipSuccess && st != s) e = hipEventRecord(ss->ev[1 + i], st);
  }
  for (int i = 0; i < nsub && e == hipSuccess; ++i) {
    if (st != s) e = hipStreamWaitEvent(s, ss->ev[1 + i], 0);
    gdn::ReadoutArgs ro;
    ro.q = x.q; ro.o = x.o; ro.snap = msnap; ro.norm_part = nullptr; ro.norms = x.norms;
    ro.BH = BH; ro.T = T; ro.S = d->S; ro.t0 = bnd[i]; ro.Tc = bnd[i + 1] - bnd[i];
    ro.Fs = T + 1; ro.f0 = 1 + bnd[i]; ro.fp8 = 0;
    if (e == hipSuccess)
      e = launch_timed(timed, GDN_KERNEL_READOUT, s, [&] { return gdn::launch_readout(D, true, ro, s); });
  }
  if (e != hipSuccess) {
    if (ss) {
      const int last = kStateSplit + 1;
      if (hipEventRecord(ss->ev[last], ss->stream) == hipSuccess) (void)hipStreamWaitEvent(s, ss->ev[last], 0);
    }
    return fail(GDN_ERR_HIP, "training forward launch: %s", hipGetErrorString(e));
  }
  return GDN_OK;
}

// The backward after its argument check.  `saved` (a training forward's
// buffer) or nullptr: then G_t, B_t and the state snapshots are replayed
// into the workspace first.
gdn_status run_backward(const gdn_desc* d, const void* q, const void* k, const void* v, const float* gamma,
                        const float* beta, const float* state_in, const void* d_out, const float* d_state_out,
                        void* dq, void* dk, void* dv, float* d_gamma, float* d_beta, float* d_state_in,
                        unsigned char* ws, const unsigned char* saved, hipStream_t s) {
  const BackwardPlan b = make_backward_plan(d, saved != nullptr);
  const int BH = (int)b.bh, T = d->T, D = d->D;
  const double c = 1.0 / std::sqrt((double)D * (double)d->S);
  const bool timed = (d->flags & GDN_FLAG_TIME_KERNELS) != 0;
  const SavedPlan sp = make_saved_plan(d);
  void* gfr = saved ? (void*)(saved + sp.gfr) : (void*)(ws + b.gfr);
  void* bfr = saved ? (void*)(saved + sp.bfr) : (void*)(ws + b.bfr);
  void* msnap = saved ? (void*)(saved + sp.msnap) : (void*)(ws + b.msnap);
  float* carrier = (float*)(ws + b.carrier);
  hipError_t e = hipSuccess;
  if (!saved) {
    e = gdn::launch_state_snapshot(state_in, msnap, BH, D, (size_t)(T + 1) * b.sfb, s);
    // forward replay: G_t and B_t for every frame
    gdn::GramArgs ga;
    ga.k = k; ga.v = v; ga.gfr = gfr; ga.bfr = bfr;
    ga.BH = BH; ga.T = T; ga.S = d->S; ga.t0 = 0; ga.Tc = T;
    ga.kscale = (float)c; ga.kscale2 = (float)(c * c); ga.fp8 = 0;
    if (e == hipSuccess) e = launch_timed(timed, GDN_KERNEL_GRAM, s, [&] { return gdn::launch_gram(D, ga, s); });
  }

  // The two serial passes run on a side stream in frame sub-ranges, next to
  // the HBM-bound passes over the tokens on the caller's stream (as in the
  // forward): the state replay (M_t snapshots, frames first to last) next to
  // C_t/dQ of the sub-range before, then the adjoint (Lambda_t, frames last
  // to first, sub-ranges mirrored so the first one is short) next to
  // dV/dK of the sub-range after.  State and adjoint travel between
  // launches through the fp32 carrier.
  int bnd[kStateSplit + 1];
  const int nsub = split_frames(T, bnd);
  SideStream* ss = nullptr;
  hipStream_t st = s;
  if (e == hipSuccess && nsub > 1) {
    e = side_stream(&ss);
    if (e == hipSuccess) {
      st = ss->stream;
      e = hipEventRecord(ss->ev[0], s);
      if (e == hipSuccess) e = hipStreamWaitEvent(st, ss->ev[0], 0);
    }
  }
  for (int i = 0; i < nsub && e == hipSuccess && !saved; ++i) {
    gdn::StateArgs sa;
    sa.gfr = gfr; sa.bfr = bfr; sa.gamma = gamma; sa.beta = beta;
    sa.state_src = i == 0 ? state_in : carrier;
    sa.state_dst = i == nsub - 1 ? nullptr : carrier;
    sa.snap = msnap;
    sa.BH = BH; sa.T = T; sa.t0 = bnd[i]; sa.Tc = bnd[i + 1] - bnd[i]; sa.Fs = T; sa.f0 = bnd[i];
    sa.beta_mode = d->beta_mode;
    sa.snap_Fs = T + 1; sa.snap_f0 = 1 + bnd[i];     // slot t+1 holds M_t
    e = launch_timed(timed, GDN_KERNEL_STATE, st, [&] { return gdn::launch_state(D, sa, st); });
    if (e == hipSuccess && st != s) e = hipEventRecord(ss->ev[1 + i], st);
  }
  // C_t = ReLU(Q_t)^T dO_t and dQ_t in one pass over Q and dO: per state
  // sub-range after a replay, else in one launch
  for (int i = 0; i < (saved ? 1 : nsub) && e == hipSuccess; ++i) {
    if (st != s && !saved) e = hipStreamWaitEvent(s, ss->ev[1 + i], 0);
    gdn::CdqArgs ca;
    ca.q = q; ca.dout = d_out; ca.msnap = msnap; ca.cfr = ws + b.cfr; ca.dq = dq; ca.BH = BH; ca.T = T;
    ca.S = d->S; ca.t0 = saved ? 0 : bnd[i]; ca.Tc = saved ? T : bnd[i + 1] - bnd[i];
    if (e == hipSuccess)
      e = launch_timed(timed, GDN_KERNEL_BACKWARD, s, [&] { return gdn::launch_cdq(D, ca, s); });
  }
  // the adjoint needs every C_t
  if (e == hipSuccess && st != s) {
    e = hipEventRecord(ss->ev[0], s);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, ss->ev[0], 0);
  }
  for (int j = 0; j < nsub && e == hipSuccess; ++j) {
    gdn::AdjointArgs aa;
    aa.gfr = gfr; aa.bfr = bfr; aa.cfr = ws + b.cfr; aa.msnap = msnap;
    aa.gamma = gamma; aa.beta = beta; aa.dstate_out = d_state_out;
    aa.lam_src = j == 0 ? nullptr : carrier;
    aa.lam_dst = j == nsub - 1 ? d_state_in : carrier;
    aa.lsnap = ws + b.lsnap; aa.part = (float*)(ws + b.part);
    aa.BH = BH; aa.T = T; aa.beta_mode = d->beta_mode;
    aa.t_hi = T - bnd[j]; aa.t_lo = T - bnd[j + 1];
    e = launch_timed(timed, GDN_KERNEL_BACKWARD, st, [&] { return gdn::launch_adjoint(D, aa, st); });
    if (e == hipSuccess && st != s) e = hipEventRecord(ss->ev[1 + j], st);
  }
  // dV and dK in one pass over K and V (Z_t formed inside)
  for (int j = 0; j < nsub && e == hipSuccess; ++j) {
    const int t_lo = T - bnd[j + 1], tc = bnd[j + 1] - bnd[j];
    if (st != s) e = hipStreamWaitEvent(s, ss->ev[1 + j], 0);
    if (e == hipSuccess && (dv || dk)) {
      gdn::DvkArgs da;
      da.k = k; da.v = v; da.lsnap = ws + b.lsnap; da.msnap = msnap; da.gamma = gamma; da.beta = beta;
      da.dv = dv; da.dk = dk; da.BH = BH; da.T = T; da.S = d->S; da.beta_mode = d->beta_mode;
      da.kscale = (float)c; da.t0 = t_lo; da.Tc = tc;
      e = launch_timed(timed, GDN_KERNEL_BACKWARD, s, [&] { return gdn::launch_dvdk(D, da, s); });
    }
  }
  if (e == hipSuccess && (d_gamma || d_beta))
    e = gdn::launch_adjoint_reduce((const float*)(ws + b.part), gamma, beta, d_gamma, d_beta, BH, T, D,
                                   d->beta_mode, s);
  if (e != hipSuccess) {
    // keep the caller's stream ordered after anything already on the side stream
    if (ss) {
      const int last = kStateSplit + 1;
      if (hipEventRecord(ss->ev[last], ss->stream) == hipSuccess) (void)hipStreamWaitEvent(s, ss->ev[last], 0);
    }
    return fail(GDN_ERR_HIP, "backward kernel launch: %s", hipGetErrorString(e));
  }
  return GDN_OK;
}

// The checks of gdn_check_args; with_workspace = false leaves the workspace
// out (a caller that has none yet checks the tensors first).
gdn_status check_io(const gdn_desc* d, const void* q, const void* k, const void* v, const float* gamma,
                    const float* beta, const float* state_in, const void* o, const float* state_out,
                    const float* state_norms, const void* workspace, size_t workspace_bytes, int state_in_required,
                    bool with_workspace) {
  g_last_error.clear();
  gdn_status st = check_desc(d);
  if (st != GDN_OK) return st;
  if (!q || !k || !v) return fail(GDN_ERR_NULL, "q, k and v are required");
  if (!gamma || !beta) return fail(GDN_ERR_NULL, "gamma and beta are required");
  if (!o) return fail(GDN_ERR_NULL, "o is required");
  if (state_in_required && !state_in) return fail(GDN_ERR_NULL, "gdn_frame_step requires state_in");
  if (!with_workspace) {
    workspace = nullptr;
    workspace_bytes = 0;
  } else if (!workspace) {
    return fail(GDN_ERR_WORKSPACE, "workspace is required (gdn_workspace_size)");
  }
  const Plan p = make_plan(d);
  if (with_workspace && workspace_bytes < ws_bytes_for(p, 1))
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes < minimum %zu", workspace_bytes, ws_bytes_for(p, 1));
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16))
    return fail(GDN_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (misaligned(gamma, 4) || misaligned(beta, 4) || misaligned(state_in, 4) || misaligned(state_out, 4) ||
      misaligned(state_norms, 4))
    return fail(GDN_ERR_ALIGN, "gamma, beta, states and norms must be 4-byte aligned");
  if (misaligned(workspace, kAlign)) return fail(GDN_ERR_ALIGN, "workspace must be 256-byte aligned");

  struct Buf { const void* p; size_t n; const char* name; };
  const Buf ins[] = {{q, p.io_bytes, "q"}, {k, p.io_bytes, "k"}, {v, p.io_bytes, "v"},
                     {gamma, p.gb_bytes, "gamma"}, {beta, p.gb_bytes, "beta"},
                     {state_in, p.state_bytes, "state_in"}};
  const Buf outs[] = {{o, p.io_bytes, "o"}, {state_out, p.state_bytes, "state_out"},
                      {state_norms, p.gb_bytes, "state_norms"}, {workspace, workspace_bytes, "workspace"}};
  for (const Buf& x : outs) {
    if (!x.p) continue;
    for (const Buf& y : ins) {
      if (x.p == state_out && y.p == state_in && state_out == state_in) continue;  // in place
      if (overlap(x.p, x.n, y.p, y.n)) return fail(GDN_ERR_ALIAS, "%s overlaps %s", x.name, y.name);
    }
    for (const Buf& y : outs)
      if (&y != &x && y.p && overlap(x.p, x.n, y.p, y.n))
        return fail(GDN_ERR_ALIAS, "%s overlaps %s", x.name, y.name);
  }
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(gdn_status s) {
  // A C caller may pass any int: read the bits, not the enum (a value outside
  // the enumerators' range is not a valid C++ value of the type).
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: a size is out of range";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unknown io_dtype or beta_mode";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: a pointer is misaligned";
    case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: forbidden buffer overlap";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: head dim or flags not supported";
    case GDN_ERR_ABI: return "GDN_ERR_ABI: ABI version mismatch";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: HIP runtime error";
  }
  return "unknown gdn_status";
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

size_t gdn_workspace_min_size(const gdn_desc* d) {
  if (check_desc(d) != GDN_OK) return 0;
  return ws_bytes_for(make_plan(d), 1);
}

size_t gdn_workspace_size(const gdn_desc* d) {
  if (check_desc(d) != GDN_OK) return 0;
  const Plan p = make_plan(d);
  const FusedPlan f = p.gram ? make_fused_plan(d) : FusedPlan();
  if (f.ok) return std::max(f.total, ws_bytes_for(p, 1));
  const size_t frames = std::min<size_t>((size_t)d->T, (size_t)kMaxFramesPerLaunch);
  return ws_bytes_for(p, frames);
}

gdn_status gdn_check_args(const gdn_desc* d, const void* q, const void* k, const void* v,
                          const float* gamma, const float* beta, const float* state_in,
                          const void* o, const float* state_out, const float* state_norms,
                          const void* workspace, size_t workspace_bytes, int state_in_required) {
  return check_io(d, q, k, v, gamma, beta, state_in, o, state_out, state_norms, workspace, workspace_bytes,
                  state_in_required, true);
}

gdn_status gdn_frame_forward(const gdn_desc* d, const void* q, const void* k, const void* v,
                             const float* gamma, const float* beta, const float* state_in,
                             void* o, float* state_out, float* state_norms,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return run(d, q, k, v, gamma, beta, state_in, o, state_out, state_norms, workspace, workspace_bytes,
             stream, 0);
}

gdn_status gdn_frame_step(const gdn_desc* d, const void* q, const void* k, const void* v,
                          const float* gamma, const float* beta, const float* state_in,
                          void* o, float* state_out, float* state_norms,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return run(d, q, k, v, gamma, beta, state_in, o, state_out, state_norms, workspace, workspace_bytes,
             stream, 1);
}

gdn_status gdn_frame_forward_noalloc(const gdn_desc* d, const void* q, const void* k, const void* v,
                                     const float* gamma, const float* beta, const float* state_in, void* o,
                                     float* state_out, float* state_norms, void* stream) {
  g_last_error.clear();
  gdn_status st = check_desc(d);
  if (st != GDN_OK) return st;
  if (d->flags & GDN_FLAG_TIME_KERNELS)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_frame_forward_noalloc records no kernel times (their events are created "
                                     "on demand)");
  const Plan p = make_plan(d);
  const FusedPlan f = p.gram ? make_fused_plan(d) : FusedPlan();
  const size_t need = f.ok ? f.total : ws_bytes_for(p, 1);
  if (need > gdn::kNoAllocScratchBytes)
    return fail(GDN_ERR_WORKSPACE, "this shape needs %zu bytes of scratch; the static scratch holds %zu", need,
                gdn::kNoAllocScratchBytes);
  // the tensors, before the scratch address is asked for (that touches the device)
  st = check_io(d, q, k, v, gamma, beta, state_in, o, state_out, state_norms, nullptr, 0, 0, false);
  if (st != GDN_OK) return st;
  void* scratch = nullptr;
  const hipError_t e = gdn::noalloc_scratch(&scratch);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "static scratch address: %s", hipGetErrorString(e));
  // the three-launch form, when it runs here, stays on `stream` (no side stream to create)
  return run(d, q, k, v, gamma, beta, state_in, o, state_out, state_norms, scratch, gdn::kNoAllocScratchBytes,
             stream, 0, false);
}

gdn_status gdn_kernel_times(double ms_out[GDN_KERNEL_SLOTS], int64_t launches_out[GDN_KERNEL_SLOTS],
                            int reset) {
  std::vector<TimedKernel> todo;
  {
    std::lock_guard<std::mutex> lk(g_time_mu);
    todo.swap(g_timed);
  }
  gdn_status st = GDN_OK;
  double ms_add[GDN_KERNEL_SLOTS] = {};
  int64_t n_add[GDN_KERNEL_SLOTS] = {};
  for (TimedKernel& tk : todo) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(tk.ev[1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, tk.ev[0], tk.ev[1]);
    if (e == hipSuccess) {
      ms_add[tk.slot] += ms;
      n_add[tk.slot] += 1;
    } else {
      st = fail(GDN_ERR_HIP, "kernel timing: %s", hipGetErrorString(e));
    }
    give_timing_event(tk.ev[0]);
    give_timing_event(tk.ev[1]);
  }
  std::lock_guard<std::mutex> lk(g_time_mu);
  for (int i = 0; i < GDN_KERNEL_SLOTS; ++i) {
    g_time_ms[i] += ms_add[i];
    g_time_n[i] += n_add[i];
    if (ms_out) ms_out[i] = g_time_ms[i];
    if (launches_out) launches_out[i] = g_time_n[i];
    if (reset) { g_time_ms[i] = 0.0; g_time_n[i] = 0; }
  }
  return st;
}

size_t gdn_backward_workspace_size(const gdn_desc* d) {
  if (check_desc(d) != GDN_OK || d->io_dtype != GDN_BF16 || (d->flags & GDN_FLAG_DIRECT) ||
      d->T > kMaxFramesPerLaunch)
    return 0;
  return make_backward_plan(d).total;
}

gdn_status gdn_frame_backward(const gdn_desc* d, const void* q, const void* k, const void* v,
                              const float* gamma, const float* beta, const float* state_in,
                              const void* d_out, const float* d_state_out,
                              void* dq, void* dk, void* dv, float* d_gamma, float* d_beta, float* d_state_in,
                              void* workspace, size_t workspace_bytes, void* stream) {
  const gdn_status status = check_backward(d, q, k, v, gamma, beta, state_in, d_out, d_state_out, dq, dk, dv,
                                           d_gamma, d_beta, d_state_in, workspace, workspace_bytes);
  if (status != GDN_OK) return status;
  return run_backward(d, q, k, v, gamma, beta, state_in, d_out, d_state_out, dq, dk, dv, d_gamma, d_beta,
                      d_state_in, (unsigned char*)workspace, nullptr, (hipStream_t)stream);
}

size_t gdn_saved_size(const gdn_desc* d) {
  if (check_desc(d) != GDN_OK || d->io_dtype != GDN_BF16 || (d->flags & GDN_FLAG_DIRECT) ||
      d->T > kMaxFramesPerLaunch)
    return 0;
  return make_saved_plan(d).total;
}

size_t gdn_backward_saved_workspace_size(const gdn_desc* d) {
  if (gdn_saved_size(d) == 0) return 0;
  return make_backward_plan(d, true).total;
}

gdn_status gdn_frame_forward_train(const gdn_desc* d, const void* q, const void* k, const void* v,
                                   const float* gamma, const float* beta, const float* state_in, void* o,
                                   float* state_out, float* state_norms, void* saved, size_t saved_bytes,
                                   void* stream) {
  // the forward's own checks, with the saved buffer in the workspace's place
  const gdn_status st = gdn_check_args(d, q, k, v, gamma, beta, state_in, o, state_out, state_norms, saved,
                                       saved_bytes, 0);
  if (st != GDN_OK) return st;
  if (d->io_dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "the training forward takes bf16 I/O only");
  if (d->flags & GDN_FLAG_DIRECT) return fail(GDN_ERR_UNSUPPORTED, "the training forward runs the Gram pipeline");
  if (d->T > kMaxFramesPerLaunch)
    return fail(GDN_ERR_UNSUPPORTED, "the training forward takes at most %d frames per call", kMaxFramesPerLaunch);
  const size_t need = make_saved_plan(d).total;
  if (saved_bytes < need) return fail(GDN_ERR_WORKSPACE, "saved buffer of %zu bytes < required %zu", saved_bytes, need);
  const Ptrs x{q, k, v, gamma, beta, state_in, o, state_out, state_norms};
  return run_train(d, x, (unsigned char*)saved, (hipStream_t)stream);
}

gdn_status gdn_frame_backward_saved(const gdn_desc* d, const void* q, const void* k, const void* v,
                                    const float* gamma, const float* beta, const void* saved, size_t saved_bytes,
                                    const void* d_out, const float* d_state_out, void* dq, void* dk, void* dv,
                                    float* d_gamma, float* d_beta, float* d_state_in, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  const gdn_status status = check_backward(d, q, k, v, gamma, beta, nullptr, d_out, d_state_out, dq, dk, dv,
                                           d_gamma, d_beta, d_state_in, workspace, workspace_bytes, saved,
                                           saved_bytes, true);
  if (status != GDN_OK) return status;
  return run_backward(d, q, k, v, gamma, beta, nullptr, d_out, d_state_out, dq, dk, dv, d_gamma, d_beta,
                      d_state_in, (unsigned char*)workspace, (const unsigned char*)saved, (hipStream_t)stream);
}

gdn_status gdn_attention_check_args(const gdn_attn_desc* d, const void* q, const void* k, const void* v,
                                    const void* o, const void* workspace, size_t workspace_bytes) {
  return check_attn(d, q, k, v, o, workspace, workspace_bytes);
}

size_t gdn_attention_workspace_size(const gdn_attn_desc* d) {
  if (check_attn_desc(d) != GDN_OK) return 0;
  return gdn::attn_split_bytes(d->D, d->B * d->H, d->Tq, d->S, attn_parts(d));
}

gdn_status gdn_attention_forward(const gdn_attn_desc* d, const void* q, const void* k, const void* v, void* o,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  const gdn_status st = check_attn(d, q, k, v, o, workspace, workspace_bytes);
  if (st != GDN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  gdn::AttnArgs aa;
  aa.q = q; aa.k = k; aa.v = v; aa.o = o;
  aa.BH = d->B * d->H; aa.Tq = d->Tq; aa.Tk = d->Tk; aa.S = d->S; aa.chunk = d->chunk;
  const double scale = d->scale != 0.f ? (double)d->scale : 1.0 / std::sqrt((double)d->D);
  aa.scale_log2 = (float)(scale * 1.4426950408889634);   // log2(e)
  // split the keys when a workspace for it came in
  aa.split = 1; aa.split_tiles = 0x7fffffff; aa.part_o = nullptr; aa.part_ml = nullptr;
  if (workspace) {
    const int parts = attn_parts(d);
    const size_t need = gdn::attn_split_bytes(d->D, aa.BH, d->Tq, d->S, parts);
    if (parts > 1 && workspace_bytes >= need) {
      const long long Nq = (long long)d->Tq * d->S;
      aa.split = parts;
      aa.split_tiles = gdn::attn_split_tiles(d->Tq, d->Tk, d->S, d->chunk, parts);
      aa.part_o = (float*)workspace;
      aa.part_ml = (float*)((unsigned char*)workspace + (size_t)parts * aa.BH * Nq * d->D * 4);
    }
  }
  const bool timed = (d->flags & GDN_FLAG_TIME_KERNELS) != 0;
  const hipError_t e = launch_timed(timed, GDN_KERNEL_ATTN, s, [&] { return gdn::launch_attn(d->D, aa, s); });
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return GDN_OK;
}

gdn_status gdn_tconv_check_args(const gdn_tconv_desc* d, const void* x, const float* w, const float* bias,
                                const void* cache_in, const void* y, const void* cache_out) {
  return check_tconv(d, x, w, bias, cache_in, y, cache_out);
}

gdn_status gdn_tconv_forward(const gdn_tconv_desc* d, const void* x, const float* w, const float* bias,
                             const void* cache_in, void* y, void* cache_out, void* stream) {
  const gdn_status st = check_tconv(d, x, w, bias, cache_in, y, cache_out);
  if (st != GDN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  gdn::TconvArgs ta;
  ta.x = x; ta.w = w; ta.bias = bias; ta.cache_in = cache_in; ta.y = y; ta.cache_out = cache_out;
  ta.B = d->B; ta.T = d->T; ta.S = d->S; ta.C = d->C; ta.chunk = d->chunk; ta.f32 = d->io_dtype == GDN_F32;
  const bool timed = (d->flags & GDN_FLAG_TIME_KERNELS) != 0;
  const hipError_t e = launch_timed(timed, GDN_KERNEL_TCONV, s, [&] { return gdn::launch_tconv(ta, s); });
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "temporal convolution launch: %s", hipGetErrorString(e));
  return GDN_OK;
}

}  // extern "C"
