// C ABI plumbing: status strings, per-thread error text, device check, workspace
// clearing.
#include <algorithm>
#include <initializer_list>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "qg_host.h"

namespace qg {

static thread_local char g_err[512] = "";

qg_status fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return (qg_status)status;
}

void clear_error() { g_err[0] = 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device verdict cache: 0 unknown, 1 gfx950, 2 other.
static int g_dev_ok[64];
static int g_dev_cus[64];
static std::mutex g_dev_mu;

qg_status check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QG_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(QG_ERR_DEVICE, "device index %d out of range", dev);
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (g_dev_ok[dev] == 0) {
            hipDeviceProp_t prop;
            e = hipGetDeviceProperties(&prop, dev);
            if (e != hipSuccess) return fail(QG_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
            g_dev_ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
            g_dev_cus[dev] = prop.multiProcessorCount;
        }
        if (g_dev_ok[dev] != 1) return fail(QG_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    }
    return QG_OK;
}

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    return g_dev_cus[dev] > 0 ? g_dev_cus[dev] : 1;
}

qg_status launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
    return QG_OK;
}

static thread_local qg_launch_override g_override = {};

const qg_launch_override& launch_override() { return g_override; }

}  // namespace qg

__global__ void qg_zero_kernel(uint4* __restrict__ p, size_t n16, uint8_t* __restrict__ tail, int ntail) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

extern "C" {

int qg_abi_version(void) { return QG_ABI_VERSION; }

const char* qg_status_string(int s) {
    switch (s) {
        case QG_OK: return "ok";
        case QG_ERR_NULL: return "null pointer";
        case QG_ERR_SHAPE: return "invalid shape";
        case QG_ERR_ALIGN: return "pointer not 16-byte aligned";
        case QG_ERR_WORKSPACE: return "workspace missing or too small";
        case QG_ERR_DEVICE: return "HIP device error";
        case QG_ERR_UNSUPPORTED: return "unsupported device (gfx950 required)";
        default: return "unknown status";
    }
}

const char* qg_last_error(void) { return qg::g_err; }

qg_status qg_set_launch_override(const qg_launch_override* o) {
    qg::clear_error();
    if (!o) {
        qg::g_override = qg_launch_override{};
        return QG_OK;
    }
    const qg_launch_override& v = *o;
    auto in = [](int x, std::initializer_list<int> ok) {
        if (x == 0) return true;
        for (int k : ok)
            if (x == k) return true;
        return false;
    };
    if (!in(v.gemv_waves, {1, 2, 4, 8}))
        return (qg_status)qg::fail(QG_ERR_SHAPE, "gemv_waves=%d not in {0, 1, 2, 4, 8}", v.gemv_waves);
    if (!in(v.smalln_form,
            {QG_FORM_SMALLN_REGS, QG_FORM_SMALLN_LDS, QG_FORM_SMALLN_LDS1, QG_FORM_SMALLN_DOT, QG_FORM_SMALLN_STREAM,
             QG_FORM_SMALLN_WALK, QG_FORM_SMALLN_SPLIT, QG_FORM_SMALLN_SLICE}))
        return (qg_status)qg::fail(QG_ERR_SHAPE, "smalln_form=%d unknown", v.smalln_form);
    if (!in(v.smalln_waves, {1, 2, 4, 8}))
        return (qg_status)qg::fail(QG_ERR_SHAPE, "smalln_waves=%d not in {0, 1, 2, 4, 8}", v.smalln_waves);
    if (!in(v.smalln_tiles, {1, 2, 4}))
        return (qg_status)qg::fail(QG_ERR_SHAPE, "smalln_tiles=%d not in {0, 1, 2, 4}", v.smalln_tiles);
    if (!in(v.smalln_depth, {2, 3, 4}))
        return (qg_status)qg::fail(QG_ERR_SHAPE, "smalln_depth=%d not in {0, 2, 3, 4}", v.smalln_depth);
    if (!in(v.verify_form, {QG_FORM_VERIFY_MFMA, QG_FORM_VERIFY_DOT, QG_FORM_VERIFY_STREAM}))
        return (qg_status)qg::fail(QG_ERR_SHAPE, "verify_form=%d unknown", v.verify_form);
    if (!in(v.verify_waves, {1, 4, 8}))
        return (qg_status)qg::fail(QG_ERR_SHAPE, "verify_waves=%d not in {0, 1, 4, 8}", v.verify_waves);
    if (!in(v.verify_tiles, {1, 2, 4}))
        return (qg_status)qg::fail(QG_ERR_SHAPE, "verify_tiles=%d not in {0, 1, 2, 4}", v.verify_tiles);
    qg::g_override = v;
    return QG_OK;
}

qg_status qg_get_launch_override(qg_launch_override* o) {
    qg::clear_error();
    if (!o) return (qg_status)qg::fail(QG_ERR_NULL, "NULL pointer");
    *o = qg::g_override;
    return QG_OK;
}

size_t qg_q4k_bytes(int64_t M, int64_t K) {
    if (M < 1 || K < 256 || K % 256) return 0;
    return (size_t)M * (size_t)(K / 256) * 144u;
}

size_t qg_q8_0_bytes(int64_t M, int64_t K) {
    if (M < 1 || K < 32 || K % 32) return 0;
    return (size_t)M * (size_t)(K / 32) * 34u;
}

qg_status qg_workspace_clear(void* ws, size_t bytes, qg_stream_t stream) {
    qg::clear_error();
    if (bytes == 0) return QG_OK;
    if (!ws) return qg::fail(QG_ERR_NULL, "workspace is NULL");
    if (!qg::aligned16(ws)) return qg::fail(QG_ERR_ALIGN, "workspace not 16-byte aligned");
    qg_status st = qg::check_device();
    if (st) return st;
    size_t n16 = bytes / 16;
    int ntail = (int)(bytes % 16);
    int blocks = (int)std::min<size_t>(std::max<size_t>(qg::ceil_div((int64_t)n16, 256), 1), 4096);
    hipLaunchKernelGGL(qg_zero_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint4*)ws, n16,
                       (uint8_t*)ws + n16 * 16, ntail);
    return qg::launch_status("qg_workspace_clear");
}

}  // extern "C"
