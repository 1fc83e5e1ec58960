// Process-wide tuning knobs of the kernel planners (set through
// im2win_set_knob in the C ABI). Every knob reads 0 by default, meaning "the
// planner's choice"; other values force a variant for tests and the ablation
// study. They change which kernel or tiling runs, never the results beyond
// the fp32 summation order, and never a workspace size. Reads and writes are
// relaxed atomics: a call that overlaps a change sees either value.
#pragma once

#include <atomic>

namespace im2win {

enum Knob : int {
    KNOB_F32_VALU = 0,       // 1: fp32 on the vector-ALU kernel
    KNOB_F32_NW,             // 4, 8, 12: waves per workgroup of the fp32 matrix kernel
    KNOB_F32_WCO,            // 1..4: 32-channel blocks per tile of the fp32 matrix kernel
    KNOB_F32_CB,             // >= 1: input channels per stage of the fp32 matrix kernel
    KNOB_F32_KSPLIT,         // 1: no K split; n > 1: K split over n waves of a workgroup
    KNOB_F32_OCC,            // >= 1: workgroups per CU of the fp32 matrix kernel
    KNOB_F16_ROWS,           // -1: row-staged fp16 kernel off
    KNOB_F16_ROWS_NWV,       // 4, 8: waves per workgroup of the row-staged kernel
    KNOB_F16_ROWS_BUFS,      // 2, 3: stage buffers of the row-staged kernel
    KNOB_F16_THIN,           // -1: thin-layer fp16 kernel off
    KNOB_F16_THIN_NB,        // 2, 4: pixel blocks per wave of the thin-layer kernel
    KNOB_F16_WIDE,           // -1: wide-tile fp16 kernel off; 1: also below 128 channels
    KNOB_F16_WIDE_NW,        // 4, 8: waves per workgroup of the wide-tile kernel
    KNOB_F16_WPX,            // 1, 2, 4, 8: waves along pixels, channel-interleaved kernel
    KNOB_F16_NWH,            // >= 1: filter stages per channel group, channel-interleaved kernel
    KNOB_TILE_ORDER,         // 1: tiles in launch order (default: XCD-grouped where a kernel has it)
    KNOB_F16_REUSE,          // -1: row-reuse fp16 kernel off (the row-staged kernel takes its shapes)
    KNOB_F16_WS,             // -1: staged fp16 kernel over the materialised tensor off
    KNOB_SYNC_STAGING,       // 1: each stage copied through registers and waited for before its
                             //    MFMAs (no copy in flight during them; no direct global-to-LDS loads)
    KNOB_F32_SMALL,          // -1: small-problem fp32 kernel off (K split across a workgroup instead)
    KNOB_F16_RES,            // -1: resident-input fp16 kernel off (prepacked calls it takes run on the
                             //     wide-tile or channel-interleaved kernel)
    KNOB_COUNT
};

// Names in the order of the enum (the C ABI's im2win_knob_name).
extern const char* const kKnobNames[KNOB_COUNT];

extern std::atomic<int> g_knobs[KNOB_COUNT];

inline int knob(Knob k) { return g_knobs[k].load(std::memory_order_relaxed); }

}  // namespace im2win
