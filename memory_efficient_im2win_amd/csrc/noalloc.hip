// The fused fp16 convolution with its filter scratch in library-owned device
// memory, for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// conv2d_im2win_fp16_fused takes a caller workspace for the prepacked
// filter; this entry point keeps it instead in `scratch`, a fixed array of
// kScratchBytes in every device's global memory, held until the process
// ends. Host code never passes the array's name to a kernel (in host code it
// names a host-side stand-in): the first call on each device, with that
// device current, looks the array's device address up with
// hipGetSymbolAddress and keeps it per device, and every launch takes that
// address. Nothing here allocates memory. Every call on a device shares its
// array and leaves the last call's prepacked filter in it; the filter packs
// write every byte the kernels read, so nothing needs clearing. Calls that
// overlap on one device (different streams, or threads) race on the array.
#include <mutex>
#include <stdint.h>

#include "im2win.h"
#include "kernels.hpp"

namespace {

using im2win::ConvShape;

constexpr size_t kScratchBytes = size_t(4) << 20;   // 4 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_addr[kMaxDevices];

// The device address of `scratch` on the current device (looked up once per
// device); nullptr if the lookup fails.
void* scratch_address()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_addr[dev] = p;
    }
    return g_addr[dev];
}

int status_of(int rc)
{
    if (rc == 0) return IM2WIN_OK;
    if (rc == -1) return IM2WIN_EINVAL;
    return IM2WIN_ELAUNCH;
}

}  // namespace

extern "C" {

int conv2d_im2win_fp16_fused_noalloc(const uint16_t* x, const uint16_t* w, float* y, int N, int Ci,
                                     int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw,
                                     void* stream)
{
    int Ho = 0, Wo = 0;
    if (!x || !w || !y) return IM2WIN_EINVAL;
    if (im2win_output_dims_strided(Hi, Wi, Hf, Wf, sh, sw, &Ho, &Wo) != IM2WIN_OK)
        return IM2WIN_EINVAL;
    const size_t need = conv2d_im2win_fp16_fused_workspace_bytes(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw);
    if (need == 0) return IM2WIN_EINVAL;            // shape outside the contract
    if (need > kScratchBytes) return IM2WIN_EWORKSPACE;
    if ((uintptr_t)x % 2 || (uintptr_t)w % 2 || (uintptr_t)y % 4) return IM2WIN_EINVAL;
    void* fws = scratch_address();
    if (!fws) return IM2WIN_ELAUNCH;
    const ConvShape c{N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo};
    hipStream_t st = static_cast<hipStream_t>(stream);
    int rc = im2win::launch_f16_filter_pack(w, fws, c, x, st);
    if (rc == -1) return status_of(im2win::launch_conv_generic_f16(x, nullptr, w, y, c, st));
    if (rc != 0) return status_of(rc);
    rc = im2win::launch_conv_f16_fused(x, w, fws, y, c, st);
    if (rc == -1) rc = im2win::launch_conv_generic_f16(x, nullptr, w, y, c, st);
    return status_of(rc);
}

}  // extern "C"
