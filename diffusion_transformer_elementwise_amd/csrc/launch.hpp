// Internal interface between the C-ABI layer (api.cpp) and the kernel files.
// Every launcher expects arguments already validated by api.cpp and returns
// the HIP status of its launch. `fast` selects the 16-byte-pack kernels (D a
// multiple of 8, every pointer 16-byte aligned, and for the modulation
// D <= RGA_RMS_MAX_D); otherwise the element-wise kernels run. dtype and
// mod_mode take the RGA_DTYPE_* and RGA_MOD_* values of rga.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace rga {

// gated residual add (gate_add.hip)
bool gate_add_grid_fits(int64_t B, int64_t L, int64_t D, int gate_mode, int es,
                        bool fast);
hipError_t launch_gate_add(const void* x, const void* u, const void* g,
                           void* out, int64_t B, int64_t L, int64_t D,
                           int gate_mode, int dtype, bool fast,
                           hipStream_t stream);

// modulation (rms_modulate.hip)
bool rms_modulate_grid_fits(int64_t B, int64_t L, int64_t D, int es, bool fast);
// wg_per_cu: see row_wg_lds (0: the library's rule)
hipError_t launch_rms_modulate(const void* x, const void* scale,
                               const void* shift, float eps, void* out,
                               int64_t B, int64_t L, int64_t D, int mod_mode,
                               int dtype, bool fast, hipStream_t stream,
                               int wg_per_cu = 0);

// modulation after a weightless LayerNorm (rms_modulate.hip); same grid
// limits as rms_modulate_grid_fits
hipError_t launch_ln_modulate(const void* x, const void* scale,
                              const void* shift, float eps, void* out,
                              int64_t B, int64_t L, int64_t D, int mod_mode,
                              int dtype, bool fast, hipStream_t stream);

// Waves per workgroup of the kernels that stage one row in LDS (binary32
// rows, long 2-byte rows; rms_modulate.hip, gate_add_rms_modulate.hip): the
// power of two from 2 to 8 nearest to one wave per 4 KB of row. Measured on
// MI355X over rows of 8 to 64 KB: fewer waves leave too few loads in flight
// per row, more leave too few rows in flight per CU (16 waves on 64 KB rows
// measured slower than 8 for binary32 rows and the fused call).
inline int lds_row_waves(int64_t row_bytes)
{
    int w = 2;
    while (w < 8 && row_bytes > 6144 * (int64_t)w)  // > 1.5 w times 4 KB
        w *= 2;
    return w;
}

// Row-modulation fast paths of the modulation and the fused call: waves (one
// row each) per workgroup, and the dynamic LDS a workgroup asks for. It
// holds the staged rows (stage_bytes: the batch's scale and shift rows, and
// a broadcast gate row for the fused call) and is raised so that about
// row_budget bytes of rows (kRowWaves per workgroup) stay on a CU: 4 to 12
// workgroups of gfx950's 160 KB of LDS per CU, each asking for a whole
// number of KB that leaves at least 1 KB of the CU unused (a request that
// fills the CU exactly could leave room for one workgroup fewer). A kernel
// that holds a row per wave streams best with few rows in flight per CU; the
// sweeps over workgroups per CU on MI355X (the bench's occupancy ablation)
// put the fast path's 8 KB modulation rows best at 5, the element path's
// realigned rows at 6-8, the fused call's fast path at 4 and its element
// path at 5-6.
constexpr int kRowWaves = 2;
constexpr int64_t kModRowBudget = 40 * 1024;        // rms/LayerNorm modulation, fast path
constexpr int64_t kModElemRowBudget = 48 * 1024;    // the same, element path
constexpr int64_t kFusedRowBudget = 32 * 1024;      // residual update + modulation
constexpr int64_t kFusedElemRowBudget = 48 * 1024;  // the same, element path
// wg_per_cu overrides the rule for measurement (rga_measure.h): > 0 asks
// for that many workgroups per CU, -1 for no cap (the staging alone).
inline int64_t row_wg_lds(int64_t row_bytes, int64_t stage_bytes, int64_t row_budget,
                          int wg_per_cu = 0)
{
    constexpr int64_t kLdsPerCu = 160 * 1024;
    if (wg_per_cu < 0)
        return stage_bytes;
    int64_t wg = wg_per_cu;
    if (wg == 0) {
        wg = (row_budget + row_bytes / 2) / row_bytes;
        wg = wg < 4 ? 4 : (wg > 12 ? 12 : wg);
    }
    const int64_t cap = ((kLdsPerCu - 1024) / wg) & ~(int64_t)1023;
    return cap > stage_bytes ? cap : stage_bytes;
}
// one workgroup's LDS limit without an opt-in attribute: larger stagings take
// the other kernels
constexpr int64_t kMaxStagedLds = 64 * 1024;

// Schedules of the row-modulation kernels that stage the batch's rows in
// LDS (the values of the RGA_SCHED_* measurement constants). The library
// runs kSchedLibrary; the others are kept for measurement
// (rga_modulate_variant, rga_fused_variant), each the same arithmetic and
// the same results in another schedule:
//   kSchedLoadsFirst  the row's loads go out before the staging loads (the
//                     modulation also reduces before the workgroup barrier)
//   kSchedOnePlus     1 + scale staged widened to binary32 (two planes)
//                     beside the shift row: no widening or add per element
//   kSchedTwoRows     two rows per wave, one after the other
//   kSchedPrefetch    two rows per wave; the second row's loads go out
//                     before the first row is worked on
enum : int {
    kSchedLibrary = 0,
    kSchedLoadsFirst = 1,
    kSchedOnePlus = 2,
    kSchedTwoRows = 3,
    kSchedPrefetch = 4,
    kSchedCount = 5
};

constexpr int sched_rows_per_wave(int sched) { return sched >= kSchedTwoRows ? 2 : 1; }

// the measurement variants run the workload's rows: bf16, D = 4096
constexpr int64_t kSchedD = 4096;
hipError_t launch_modulate_variant(const void* x, const void* scale, const void* shift,
                                   float eps, void* out, int64_t B, int64_t L, int sched,
                                   hipStream_t stream);
hipError_t launch_fused_variant(const void* x, const void* u, const void* g, const void* scale,
                                const void* shift, float eps, void* x_out, void* y, int64_t B,
                                int64_t L, int sched, hipStream_t stream);

// residual update then modulation, one pass (gate_add_rms_modulate.hip)
bool gate_add_rms_modulate_grid_fits(int64_t B, int64_t L, int64_t D, int es, bool fast);
hipError_t launch_gate_add_rms_modulate(const void* x, const void* u,
                                        const void* g, const void* scale,
                                        const void* shift, float eps,
                                        void* x_out, void* y, int64_t B,
                                        int64_t L, int64_t D, int gate_mode,
                                        int mod_mode, int dtype, bool fast,
                                        hipStream_t stream, int wg_per_cu = 0);

// tanh-GELU over [rows, F] with an optional bias row (gelu_tanh.hip); fast:
// every pointer 16-byte aligned and, with a bias, F % 8 == 0
bool gelu_tanh_grid_fits(int64_t rows, int64_t F, bool has_bias, int es, bool fast);
hipError_t launch_gelu_tanh(const void* x, const void* bias, void* out,
                            int64_t rows, int64_t F, int dtype, bool fast,
                            hipStream_t stream);

// measurement helpers (measure.hip); n16 = number of 16-byte vectors
bool stream_grid_fits(int64_t n16);
hipError_t launch_copy(const void* src, void* dst, int64_t n16,
                       hipStream_t stream);
hipError_t launch_fill(void* dst, int64_t n16, uint32_t value,
                       hipStream_t stream);
hipError_t launch_read(const void* src, int64_t n16, void* sink,
                       hipStream_t stream);
// nsrc in 0..3 source streams, dst NULL for a read-only stream (then sink is
// the 16-byte word the fold may reach), words_per_lane 1, 2 or 4
hipError_t launch_stream(const void* const* src, int nsrc, void* dst, int64_t n16,
                         int words_per_lane, void* sink, hipStream_t stream);

// bf16 broadcast-gate add in a chosen shape, for measurement (gate_add.hip):
// rows_per_wave 1, 2, 4 or 8 with the gate pack held across them, and the
// store's cache policy (RGA_STORE_* of rga_measure.h)
bool gate_add_variant_grid_fits(int64_t B, int64_t L, int64_t D, int rows_per_wave);
hipError_t launch_gate_add_variant(const void* x, const void* u, const void* g, void* out,
                                   int64_t B, int64_t L, int64_t D, int rows_per_wave,
                                   int store_policy, hipStream_t stream);

}  // namespace rga
