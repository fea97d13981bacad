// Internal interface between the host orchestration (gdn_api.cpp) and the
// HIP kernels (gdn_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdn {

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
  void* snap;               // [BH][Tc][D][D] state snapshots, transposed ([value][key])
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
  const float* norm_part;   // as in RecurArgs, or nullptr
  float* norms;             // [BH][T] or nullptr
  int BH, T, S, t0, Tc;
};

// Enqueue recurrence + readout for one range of frames.  `ev`, when not null,
// holds three events recorded before, between and after the two kernels.
hipError_t launch_chunk(int D, bool bf16, const RecurArgs& ra, const ReadoutArgs& ro,
                        hipStream_t stream, hipEvent_t* ev);

// Dynamic LDS bytes of the recurrence kernel for (D, dtype).
size_t recur_lds_bytes(int D, bool bf16);

}  // namespace gdn
