// Internal interface between the host orchestration (gdn_api.cpp) and the
// HIP kernels (gdn_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <map>
#include <mutex>

namespace gdn {

// One-time, per-device setup of a kernel launcher (function attributes,
// occupancy, CU count), safe when several host threads make their first
// call at once: the first caller on a device runs `init(dev, info)` under the
// lock; later callers get the cached result.  A failed init is not cached.
struct LaunchInfo {
  int cus = 0;     // compute units of the device
  int slots = 0;   // resident workgroups of the launcher's persistent kernel, if any
};
class DeviceOnce {
 public:
  template <class Init>
  hipError_t get(Init&& init, LaunchInfo* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(mu_);
    auto it = done_.find(dev);
    if (it == done_.end()) {
      LaunchInfo info;
      e = init(dev, info);
      if (e != hipSuccess) return e;
      it = done_.emplace(dev, info).first;
    }
    *out = it->second;
    return hipSuccess;
  }

 private:
  std::mutex mu_;
  std::map<int, LaunchInfo> done_;
};

// Frames per launch are capped so that per-frame scalars fit in LDS.
constexpr int kMaxFramesPerLaunch = 1024;

// One launch of the recurrence covers frames [t0, t0 + Tc) of the call.
struct RecurArgs {
  const void* k;            // [BH][T][S][D]
  const void* v;            // [BH][T][S][D]
  const float* gamma;       // [BH][T]
  const float* beta;        // [BH][T]
  const float* state_src;   // [BH][D][D] or nullptr (zero state)
  float* state_dst;         // [BH][D][D] or nullptr
  void* snap;               // per (head, frame) state snapshot: fp32 I/O [D][D] transposed
                            // ([value][key]); bf16 I/O D*D bf16 as blocks [jt][I] of
                            // 64 lanes x 4, lane (n, g) holding M[16I+4g+r][16jt+n]
  float* norm_part;         // [BH][Tc][D/16] or nullptr
  int units;                // BH * (D/16) workgroups with work
  int T, S, t0, Tc;
  int beta_mode;            // 0 ERASE, 1 WRITE
  float kscale;             // 1/sqrt(D*S), rounded once to fp32
};

struct ReadoutArgs {
  const void* q;            // [BH][T][S][D]
  void* o;                  // [BH][T][S][D]
  const void* snap;         // as in RecurArgs
  const float* norm_part;   // as in RecurArgs; nullptr: norms from the bf16 snapshot
  float* norms;             // [BH][T] or nullptr
  int BH, T, S, t0, Tc;
  int Fs, f0;               // snapshots (and norm partials) hold [BH][Fs] frames from f0
  int fp8;                  // 1: Q and O are OCP e4m3 bytes (bf16 snapshots only)
  int nsplit;               // workgroups per frame, each a share of its chunks (set by the launcher)
};

// C_t = ReLU(Q_t)^T dO_t and dQ_t of the backward in one pass over Q_t and dO_t.
struct CdqArgs {
  const void* q;            // [BH][T][S][D] bf16
  const void* dout;         // [BH][T][S][D] bf16
  const void* msnap;        // bf16 snapshots of M_{t-1}: [BH][T+1] (slot t+1 holds M_t)
  void* cfr;                // out: C_t in B's layout, [BH][T]
  void* dq;                 // out: [BH][T][S][D] bf16 or nullptr
  int BH, T, S;
  int t0, Tc;               // this launch's frames: t0 .. t0+Tc-1
};

// dV_t and dK_t of the backward in one pass over K_t and V_t.
struct DvkArgs {
  const void* k;            // [BH][T][S][D] bf16
  const void* v;            // [BH][T][S][D] bf16
  const void* lsnap;        // bf16 snapshots of Lambda_t: [BH][T]
  const void* msnap;        // bf16 snapshots of M_{t-1}: [BH][T+1], slot t holds M_{t-1}
  const float* gamma;       // [BH][T]
  const float* beta;        // [BH][T]
  void* dv;                 // [BH][T][S][D] bf16 or nullptr
  void* dk;                 // [BH][T][S][D] bf16 or nullptr
  int BH, T, S, beta_mode;
  float kscale;             // 1/sqrt(D*S)
  int t0, Tc;               // this launch's frames: t0 .. t0+Tc-1
};

// Block-causal temporal convolution (gdn_tconv.hip).
struct TconvArgs {
  const void* x;            // [B][T][S][C] bf16 or fp32
  const float* w;           // [3][C]: taps of the previous, current, next frame
  const float* bias;        // [C] or nullptr
  const void* cache_in;     // [B][S][C] or nullptr (zeros)
  void* y;                  // [B][T][S][C]
  void* cache_out;          // [B][S][C] or nullptr
  int B, T, S, C, chunk, f32;
  // set by launch_tconv
  int cols_per_token, seg_frames;
  long long cols;
};

// Block-causal softmax attention (gdn_attn.hip).
struct AttnArgs {
  const void* q;            // [BH][Tq*S][D] bf16 (the last Tq frames of the key sequence)
  const void* k;            // [BH][Tk*S][D] bf16
  const void* v;            // [BH][Tk*S][D] bf16
  void* o;                  // [BH][Tq*S][D] bf16
  int BH, Tq, Tk, S, chunk;
  float scale_log2;         // softmax scale times log2(e)
  // key split (split > 1): each workgroup runs split_tiles key tiles and
  // writes its unnormalised O (fp32) and (max, sum) to the partial arrays;
  // a merge kernel combines them
  int split, split_tiles;
  float* part_o;            // [split][BH][Tq*S][D] fp32
  float* part_ml;           // [split][BH][Tq*S][2] fp32: running max (log2 units), sum
};

// Gram pass (bf16 or e4m3 I/O): per (head, frame) G = Kf^T Kf and B = Kf^T V.
struct GramArgs {
  const void* k;            // [BH][T][S][D] bf16, or OCP e4m3 when fp8
  const void* v;            // [BH][T][S][D] as k
  void* gfr;                // [BH][Tc] x gram_frame_bytes(D): G as state-pass A operands
  void* bfr;                // [BH][Tc] x input_frame_bytes(D): B in accumulator layout
  int BH, T, S, t0, Tc;
  float kscale, kscale2;    // 1/sqrt(D*S) and 1/(D*S), each rounded once to fp32
  int fp8;                  // 1: K and V are OCP e4m3 bytes
  // optional (launches of at most 2 frames per CU only): BH extra
  // workgroups copy each head's [D][D] fp32 state from copy_src to copy_dst
  const float* copy_src = nullptr;
  float* copy_dst = nullptr;
};

// Chain and readout of a short chunk in one launch (see gdn_step_tail_kernel).
struct TailArgs {
  const void* q;            // [BH][T][S][D] bf16, or OCP e4m3 when fp8
  void* o;                  // as q
  const void* gfr;          // this launch's G_t: [BH][Tc] frames, as in GramArgs
  const void* bfr;          // this launch's B_t: [BH][Tc] frames
  const float* gamma;       // [BH][T]
  const float* beta;        // [BH][T]
  const float* state_src;   // [BH][D][D] fp32 or nullptr (zero state); must not alias state_dst
  float* state_dst;         // [BH][D][D] fp32 or nullptr
  int BH, T, S, t0, Tc;
  int nsplit;               // workgroups per (head, frame, value tile): shares of the frame's chunks
  int beta_mode;            // 0 ERASE, 1 WRITE
  int fp8;
};
// Longest launch (frames per head) that takes the chunk tail; each workgroup
// recomputes the chain of the frames before its own (all kTailMaxFrames of
// them, those past its own frame on zeros).
constexpr int kTailMaxFrames = 4;

// State pass (bf16 I/O): the serial frame loop over G and B.
struct StateArgs {
  const void* gfr;          // as in GramArgs
  const void* bfr;          // as in GramArgs
  const float* gamma;       // [BH][T]
  const float* beta;        // [BH][T]
  const float* state_src;   // [BH][D][D] or nullptr (zero state)
  float* state_dst;         // [BH][D][D] or nullptr
  void* snap;               // as in RecurArgs (bf16 block layout)
  int BH, T, t0, Tc;
  int Fs, f0;               // staging arrays hold [BH][Fs] frames; this launch's first frame is f0
  int beta_mode;            // 0 ERASE, 1 WRITE
  int snap_Fs, snap_f0;     // snapshot array: [BH][snap_Fs] frames, this launch's first at snap_f0
};

// Adjoint state pass of the backward: Lambda_t = dL/dM_t, frames last to first.
struct AdjointArgs {
  const void* gfr;          // G_t as in GramArgs, [BH][T] frames
  const void* bfr;          // B_t (WRITE mode only; else unused), [BH][T]
  const void* cfr;          // C_t = ReLU(Q_t)^T dO_t in B's layout, [BH][T]
  const void* msnap;        // bf16 snapshots of M_{t-1}: [BH][T+1], slot t holds M_{t-1}
  const float* gamma;       // [BH][T]
  const float* beta;        // [BH][T]
  const float* dstate_out;  // [BH][D][D] or nullptr (used when lam_src is null)
  const float* lam_src;     // [BH][D][D] Lambda_{t_hi-1} from the previous launch, or nullptr
                            // (then Lambda_{T-1} = dstate_out + C_{T-1}: t_hi must be T)
  float* lam_dst;           // [BH][D][D] or nullptr: Lambda_{t_lo-1} (dL/dM_in when t_lo = 0);
                            // may equal lam_src
  void* lsnap;              // out: bf16 snapshots of Lambda_t, [BH][T] (block layout)
  float* part;              // out: [BH][T][NB*NB][4] per-wave partial sums
  int BH, T, beta_mode;
  int t_lo, t_hi;           // this launch's frames, run from t_hi-1 down to t_lo
};

// One-launch forward (gdn_fused.hip): gram, state and readout roles of the
// Gram pipeline in one persistent cooperative launch, handing G_t, B_t and
// the bf16 states over through rings that stay in one XCD's L2.
constexpr int kFusedWaves = 4;            // waves per workgroup; two workgroups per CU
constexpr int kFusedMaxRG = 48;           // gram ring slots per head (at most)
constexpr int kFusedMaxRM = 16;           // state ring slots per head (at most)
constexpr int kFusedMaxCW = 2;            // chain workgroups per head (one per 4 value tiles)
constexpr size_t kFusedCtlTicket = 64;    // control block: abort word at 0, per-XCD tickets from here
constexpr size_t kFusedCtlCu = 2048;      // (64 bytes apart, up to 16 XCDs), then per-CU words (two
constexpr size_t kFusedCtlHead = kFusedCtlCu + 16 * 256 * 8;   // per CU id and XCD), then per-head flags
constexpr size_t kFusedCtlPerHead = 8192;
inline size_t fused_ctl_bytes(int BH) { return kFusedCtlHead + (size_t)BH * kFusedCtlPerHead; }
// per head: the chain workgroups' progress words, then gready per gram slot,
// then rdone per state slot, 64 bytes apart
static_assert((kFusedMaxCW + kFusedMaxRG + kFusedMaxRM) * 64 <= (int)kFusedCtlPerHead, "per-head flags");
size_t fused_slot_bytes(int D);           // one gram ring slot: G_t (stored blocks) and B_t

struct FusedArgs {
  const void* q;            // [BH][T][S][D] bf16, or OCP e4m3
  const void* k;
  const void* v;
  void* o;
  const float* gamma;       // [BH][T]
  const float* beta;        // [BH][T]
  const float* state_in;    // [BH][D][D] or nullptr (zero state)
  float* state_out;         // [BH][D][D] or nullptr
  float* norms;             // [BH][T] or nullptr
  unsigned char* ctl;       // fused_ctl_bytes(BH), cleared by the launcher
  unsigned char* gring;     // [BH][RG] x fused_slot_bytes(D)
  unsigned char* mring;     // [BH][RM] x D*D*2 (bf16 state, snapshot block layout)
  int BH, T, S;
  int NX;                   // XCDs; head h lives on XCD h % NX
  int RG, RM, L;            // ring slots per head; readout lag in frames (4 <= L <= RG + RM - 2, 5 <= RG)
  int balance;              // 1: the readouts of an XCD's extra head run on a less loaded XCD
  int grid;                 // workgroups (two per CU, a multiple of NX)
  float kscale, kscale2;    // 1/sqrt(D*S) and 1/(D*S), each rounded once to fp32
};
// Static device scratch of the allocation-free forward: its size, and its
// address on the current device (taken once per device with
// hipGetSymbolAddress).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** out);

// Clears the control block and launches; fp8: e4m3 I/O; erase: beta mode.
hipError_t launch_fused(int D, const FusedArgs& fa, int fp8, int erase, hipStream_t stream);

// Kernel launchers (enqueue only).  D in {16, ..., 128}.
hipError_t launch_recurrence(int D, bool bf16, const RecurArgs& ra, hipStream_t stream);
hipError_t launch_readout(int D, bool bf16, const ReadoutArgs& ro, hipStream_t stream);
hipError_t launch_gram(int D, const GramArgs& ga, hipStream_t stream);
hipError_t launch_state(int D, const StateArgs& sa, hipStream_t stream);
hipError_t launch_step_tail(int D, const TailArgs& ta, int cus, hipStream_t stream);
hipError_t launch_adjoint(int D, const AdjointArgs& aa, hipStream_t stream);
hipError_t launch_dvdk(int D, const DvkArgs& da, hipStream_t stream);
hipError_t launch_tconv(const TconvArgs& ta, hipStream_t stream);
hipError_t launch_attn(int D, const AttnArgs& aa, hipStream_t stream);
// key split chosen for a launch on the current device: how many parts, and
// the workspace bytes they need (0 when one part is best)
int attn_split_parts(int D, int BH, int Tq, int Tk, int S, int chunk, int cus);
size_t attn_split_bytes(int D, int BH, int Tq, int S, int parts);
int attn_split_tiles(int Tq, int Tk, int S, int chunk, int parts);   // key tiles per part
hipError_t launch_cdq(int D, const CdqArgs& ca, hipStream_t stream);
hipError_t launch_state_snapshot(const float* state, void* snap, int BH, int D, size_t slot_stride_bytes,
                                 hipStream_t stream);
hipError_t launch_adjoint_reduce(const float* part, const float* gamma, const float* beta, float* dgamma,
                                 float* dbeta, int BH, int T, int D, int beta_mode, hipStream_t stream);


// Workspace bytes per (head, frame) of the Gram pass outputs.
size_t gram_frame_bytes(int D);
size_t input_frame_bytes(int D);

}  // namespace gdn
