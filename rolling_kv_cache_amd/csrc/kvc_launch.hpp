// kvc_launch.hpp -- host-callable launchers of the libkvc HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>

#include "kvc_device.hpp"

namespace kvc {

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_retime(const RetimeArgs& a, int32_t nblocks, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);
// copy n int32 from pinned host memory (its device-visible address) to device memory
hipError_t launch_stage_idx(const int32_t* host_visible, int32_t* dst, int32_t n, hipStream_t s);
hipError_t launch_export(const ExportArgs& a, int32_t n_valid, hipStream_t s);
// Attention: the matrix-core path for bf16 with head_dim 128, and for bf16
// with head_dim 64 on a cache of rotated keys, else the general per-row path;
// `paths` holds kPath* bits (kPathGeneral selects the general path for any
// cache).
hipError_t launch_attend(const AttendArgs& a, uint32_t paths, hipStream_t s);
hipError_t launch_attend_mfma(const AttendArgs& a, uint32_t paths, hipStream_t s);
hipError_t launch_attend_mfma64(const AttendArgs& a, hipStream_t s);
// Scores: the matrix-core passes for bf16 with head_dim 128 or 64, else the
// general per-row/per-column path (kPathGeneral in `paths` selects the latter).
hipError_t launch_score(const ScoreArgs& a, uint32_t paths, hipStream_t s);
// MemRoPE: fold evicted frames into the EMA memories; copy the memory slots out
hipError_t launch_mem_fold(const MemFoldArgs& a, hipStream_t s);
hipError_t launch_mem_export(const MemExportArgs& a, hipStream_t s);
// frame sums, their Gram matrix, then the Relax Forcing scores
hipError_t launch_relax(const RelaxArgs& a, hipStream_t s);
// Device address of the current GPU's copy of the library-held relax scratch
// (kRelaxNoallocScratch bytes), looked up once per device.
hipError_t relax_noalloc_scratch(void** ptr);
// rows + columns passes over a query window already rotated into qbf
// ([H][Nq][128] bf16); writes a.m (log2 normaliser per row) and a.part
hipError_t launch_score_mfma(const ScoreArgs& a, const uint16_t* qbf, hipStream_t s);
// the same for bf16 head_dim 64 (qbf: [H][Nq][64])
hipError_t launch_score_mfma64(const ScoreArgs& a, const uint16_t* qbf, hipStream_t s);

}  // namespace kvc
