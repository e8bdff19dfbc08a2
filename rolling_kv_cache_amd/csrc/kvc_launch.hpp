// kvc_launch.hpp -- host-callable launchers of the libkvc HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>

#include "kvc_device.hpp"

namespace kvc {

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_retime(const RetimeArgs& a, int32_t nblocks, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);
hipError_t launch_export(const ExportArgs& a, int32_t n_valid, hipStream_t s);
// Attention: the matrix-core path for bf16 with head_dim 128, else the
// general per-row path.  `force_general` selects the latter (tests).
hipError_t launch_attend(const AttendArgs& a, hipStream_t s, bool force_general);
hipError_t launch_attend_mfma(const AttendArgs& a, hipStream_t s);
// Scores: the matrix-core passes for bf16 with head_dim 128, else the general
// per-row/per-column path (force_general selects the latter).
hipError_t launch_score(const ScoreArgs& a, hipStream_t s, bool force_general);
// MemRoPE: fold evicted frames into the EMA memories; copy the memory slots out
hipError_t launch_mem_fold(const MemFoldArgs& a, hipStream_t s);
hipError_t launch_mem_export(const MemExportArgs& a, hipStream_t s);
// frame sums, their Gram matrix, then the Relax Forcing scores
hipError_t launch_relax(const RelaxArgs& a, hipStream_t s);
// rows + columns passes over a query window already rotated into qbf
// ([H][Nq][128] bf16); writes a.m (log2 normaliser per row) and a.part
hipError_t launch_score_mfma(const ScoreArgs& a, const uint16_t* qbf, hipStream_t s);

}  // namespace kvc
