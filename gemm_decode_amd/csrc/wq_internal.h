// Internal declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/wq.h"

namespace wq {

constexpr int kGroup = 128;        // group size along K for the group-128 formats
constexpr int kMaxSplit = 32;      // largest split_k of the tuning grid
constexpr int kGemvMaxM = 7;       // tokens < 8 take the GEMV
constexpr int kGemvRowsPerWave = 4;  // output rows per GEMV workgroup tile
constexpr int kGemvMaxWaves = 16;    // waves per GEMV workgroup (intra-workgroup K split)

// Thread-local error text behind wq_last_error().
void set_error(const std::string& msg);
wq_status fail(wq_status st, const std::string& msg);
wq_status hip_fail(hipError_t e, const char* what);

#define WQ_HIP_CHECK(call)                                   \
  do {                                                       \
    hipError_t e_ = (call);                                  \
    if (e_ != hipSuccess) return ::wq::hip_fail(e_, #call);  \
  } while (0)

// Shape/format validation shared by every entry point (no device access).
wq_status check_shape(int fmt, int64_t K, int64_t N);
wq_status check_weight(const wq_weight* w, int want_layout);

// K granule that split-K slices align to: 16 (per-channel W8) or 128 (group-128).
inline int64_t split_granule(int fmt) { return fmt == WQ_FMT_W8_PC ? 16 : kGroup; }

// --- kernel launchers (implemented in the .hip files) ---
wq_status launch_pack(const float* w, const wq_weight* out, hipStream_t s);
wq_status launch_repack(const wq_weight* src, const wq_weight* dst, bool to_gfx950, hipStream_t s);
wq_status launch_gemv(const wq_weight* w, const uint16_t* x, int M, uint16_t* y, int split_k,
                      int waves, void* ws, hipStream_t s);
// Waves per GEMV workgroup when none is tuned or given.
int gemv_default_waves(int64_t K, int64_t N, int fmt, int M, int split_k);
// Largest waves per GEMV workgroup that fits the registers at this format and M.
int gemv_max_waves(int fmt, int M);
wq_status launch_gemm(const wq_weight* w, const uint16_t* x, int64_t M, uint16_t* y, int tile,
                      hipStream_t s);

// Workspace bytes for a GEMV with the given split (fp32 partials of every slice).
size_t gemv_workspace_bytes(int64_t N, int64_t M, int split_k);

// Device tag "<arch>:<CUs>" of the current device; empty on failure.
std::string current_device_tag();

}  // namespace wq
