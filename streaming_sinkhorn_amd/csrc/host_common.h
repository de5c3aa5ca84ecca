// Host-side helpers shared by the C-ABI translation units: error text,
// HIP status checks, operand layout / pass shape selection, argument and
// workspace checks.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "flashot.h"
#include "kernels.h"

namespace flashot {
namespace host {

// Records msg as the thread's last error and returns code.
int fail(int code, const std::string& msg);
const char* last_error();

#define OT_HIP(expr)                                                                     \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return ::flashot::host::fail(OT_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)


inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Kernel configuration for a point dimension / storage type.
struct KConf {
  int mode;     // 0 fp32 operands, 1 bf16, 2 fp32 as three bf16 parts, 3 as two fp16 parts
  int kbw;      // dimension values per k-block (8 fp32, 16 bf16 / split)
  int kblocks;  // k-blocks needed to cover d
  int kb;       // 1 KiB operand units per tile held in registers (3 / 2 per k-block when split)
  int kbp;      // padded operand units per tile
  bool xres;    // row operand resident in registers
  bool lds;     // column tiles shared by the workgroup's waves through LDS
  int ri;       // row tiles per wave in the LSE pass
  int ct, bk;   // tiled wide pass: column tiles per block, k-blocks per LDS stage
};

int f32_operand_mode(int32_t flags);
KConf kernel_conf(int64_t d, int bf16, int f32_mode, bool for_apply = false);
// Workgroup targets measured on MI355X: the solve's register-resident
// log-sum-exp passes run best with about 1024 workgroups (16 column splits
// at 20000 rows: 2-4.5 % faster than 32 at d = 16, 64 and 128, fp32 and
// bf16); the wide pass, the transport applications and the HVP's
// transport-vector passes with about 2048.
constexpr int kTargetWorkgroups = 2048;
constexpr int kTargetWorkgroupsResident = 1024;
// The solve's wide passes take at least 8 column splits: at n = 200000,
// m = 10000, d = 1024 (782 row groups, 79 column blocks) the 2048 target
// alone gives 3, and a log-sum-exp launch averaged 9.80-9.85 ms with 8
// against 10.37-10.40 ms with 3 (9.73-9.75 ms with 16). The floor only
// changes passes of more than 256 row groups (over 65536 rows).
constexpr int kMinSplitsWide = 8;
PassShape make_pass(int rtiles, int ctiles, const KConf& k, int ri, int forced, int max_splits,
                    int target = kTargetWorkgroups, int min_splits = 1);
// Non-resident transport passes stream whole blocks of kApplyWideCT column
// tiles: the tiles per split are rounded up to a multiple of it (the split
// count shrinks accordingly).
inline void whole_block_splits(PassShape& s) {
  s.tps = ceil_div(s.tps, kApplyWideCT) * kApplyWideCT;
  s.splits = ceil_div(s.ctiles, s.tps);
}
int check_problem(const ot_problem* p);
// ws == NULL: writes need to *ws_bytes and sets *query; otherwise checks size
// and alignment.
int check_ws(void* ws, size_t* ws_bytes, size_t need, bool* query);
// fp32 points in the two-part fp16 operand mode: waits for the range plan on
// `st` (one stream synchronisation) and returns OT_ERR_UNSUPPORTED when the
// points do not fit the fp16 parts, before the passes that read them.
int check_half2_range(const Half2Plan* plan, hipStream_t st);

}  // namespace host
}  // namespace flashot
