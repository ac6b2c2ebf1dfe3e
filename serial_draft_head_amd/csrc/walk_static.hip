// walk_static.hip -- dsw_walk_static: the walk of dsw_walk without a handle
// and without any allocation, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Its workspace -- mailboxes, launch counters, status word and
// the batched kernel's buffer of sampled logits -- is the file-scope device
// array `scratch` below, which every GPU the library runs on holds until the
// process ends.  Calls on one GPU share that GPU's array: calls that overlap
// on the device race (one at a time per GPU, as one handle serves one stream
// at a time).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dsw.h"
#include "launch.h"
#include "walk_params.h"

namespace {

constexpr size_t kWsBytes = 4u << 20;      // the workspace part (its layout needs about 3.2 MiB)
constexpr size_t kBlogBytes = 32u << 20;   // the batched kernel's sampled logits (batched_logits_bytes)
constexpr size_t kScratchBytes = kWsBytes + kBlogBytes;
constexpr int kMaxDevices = 64;
constexpr int kStaticGammaMax = 256;       // the step count every call's epochs are spaced by
constexpr unsigned kStaticFlags = DSW_FLAG_FORCE_STREAM | DSW_FLAG_COOPERATIVE | DSW_FLAG_VALU_GEMV |
                                  DSW_FLAG_MFMA_GEMV | DSW_FLAG_BATCHED | DSW_FLAG_SINGLE_ROUND;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Zeroes n16 16-byte words from p (a fill kernel, not a memset, so that a
// graph that captures it replays it as a kernel).
__global__ void __launch_bounds__(256) zero_words(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct DeviceState {
    bool ready;
    unsigned char* ptr;  // device address of `scratch` on this device (never the host-side name)
    dsw_devinfo dev;
};
std::mutex g_mu;
DeviceState g_state[kMaxDevices];

struct CurrentDevice {
    int prev = -1;
    bool ok = false;
    explicit CurrentDevice(int device) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        ok = hipSetDevice(device) == hipSuccess;
    }
    ~CurrentDevice() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

int zero_workspace(unsigned char* ptr, void* stream) {
    hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<uint4*>(ptr), kWsBytes / 16);
    return hipGetLastError() == hipSuccess ? DSW_OK : DSW_ERR_HIP;
}

// Once per device, with that device current: the device address of
// `scratch`, the device description, and a zero fill of the workspace part
// on `stream` (waited for when `wait`).
int setup(int device, void* stream, bool wait, DeviceState** out) {
    int n = 0;
    if (device < 0 || device >= kMaxDevices || hipGetDeviceCount(&n) != hipSuccess || device >= n)
        return DSW_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState& s = g_state[device];
    if (!s.ready) {
        int rc = dsw_device_info(device, &s.dev);
        if (rc) return rc;
        CurrentDevice g(device);
        if (!g.ok) return DSW_ERR_DEVICE;
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return DSW_ERR_HIP;
        s.ptr = static_cast<unsigned char*>(ptr);
        rc = zero_workspace(s.ptr, stream);
        if (rc) return rc;
        if (wait && hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return DSW_ERR_HIP;
        s.ready = true;
    }
    *out = &s;
    return DSW_OK;
}

dsw::Workspace workspace_at(unsigned char* base) {
    const dsw::WorkspaceLayout L = dsw::workspace_layout();
    dsw::Workspace ws;
    ws.mail = reinterpret_cast<unsigned long long*>(base + L.mail);
    ws.tokw = reinterpret_cast<unsigned long long*>(base + L.tokw);
    ws.round_ctr = reinterpret_cast<unsigned*>(base + L.ctl) + dsw::kCtlRound;
    ws.fam_ctr = reinterpret_cast<unsigned*>(base + L.ctl) + dsw::kCtlFam;
    ws.status = reinterpret_cast<unsigned*>(base + L.ctl) + dsw::kCtlStatus;
    ws.bkey = reinterpret_cast<unsigned long long*>(base + L.bkey);
    ws.bdec = reinterpret_cast<unsigned long long*>(base + L.bdec);
    ws.blog = reinterpret_cast<uint16_t*>(base + kWsBytes);
    return ws;
}

}  // namespace

extern "C" int dsw_static_init(int device) {
    if (dsw::workspace_layout().total > kWsBytes) return DSW_ERR_SCRATCH;
    DeviceState* s = nullptr;
    return setup(device, nullptr, true, &s);
}

extern "C" int dsw_walk_static(int device, int V, int w2_dtype, unsigned flags, const void* W1, const void* W2,
                               const float* w2_scale, const void* base, const int32_t* anchor, const float* T,
                               const float* uniforms, int32_t* tokens, void* logits, int B, int gamma,
                               void* stream) {
    if (V < 1) return DSW_ERR_VOCAB;
    if (w2_dtype != DSW_BF16 && w2_dtype != DSW_INT8) return DSW_ERR_DTYPE;
    if (flags & ~kStaticFlags) return DSW_ERR_ARG;
    if (B < 0 || B > dsw::kMaxBatch) return DSW_ERR_BATCH;
    if (gamma < 0 || gamma > kStaticGammaMax) return DSW_ERR_GAMMA;
    if (B == 0 || gamma == 0) return DSW_OK;
    if (dsw::workspace_layout().total > kWsBytes) return DSW_ERR_SCRATCH;
    DeviceState* s = nullptr;
    int rc = setup(device, stream, false, &s);
    if (rc) return rc;
    dsw_plan_info plan;
    rc = dsw_plan_compute(&s->dev, V, dsw::kRank, gamma, B, w2_dtype, flags, &plan);
    if (rc) return rc;
    // the batched kernel keeps the sampled requests' logits of the current
    // step in the caller's logits, or else in the scratch array
    if (plan.batch_tile == dsw::kMaxBatch && logits == nullptr && dsw::batched_logits_bytes(V, B) > kBlogBytes)
        return DSW_ERR_SCRATCH;
    dsw::LaunchCtx x;
    x.device = device;
    x.V = V;
    x.gamma_max = kStaticGammaMax;
    x.B_max = dsw::kMaxBatch;  // every slot a later call may read is zeroed at entry
    x.dtype = w2_dtype;
    x.flags = flags;
    x.dev = &s->dev;
    x.ws = workspace_at(s->ptr);
    x.spin_limit = dsw::kSpinLimit;
    x.skew = 0u;
    x.seeded = 0;
    x.seed = 0ull;
    x.trace = nullptr;
    x.trace_bytes = 0;
    return dsw::launch_walk(x, W1, W2, w2_scale, base, anchor, T, uniforms, tokens, logits, B, gamma, stream,
                            nullptr, nullptr);
}

extern "C" int dsw_static_status(int device) {
    int n = 0;
    if (device < 0 || device >= kMaxDevices || hipGetDeviceCount(&n) != hipSuccess || device >= n)
        return DSW_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState& s = g_state[device];
    if (!s.ready) return DSW_OK;  // nothing has run on this device
    CurrentDevice g(device);
    if (!g.ok) return DSW_ERR_DEVICE;
    if (hipDeviceSynchronize() != hipSuccess) return DSW_ERR_HIP;
    unsigned st = 0;
    const dsw::Workspace ws = workspace_at(s.ptr);
    if (hipMemcpy(&st, ws.status, sizeof st, hipMemcpyDeviceToHost) != hipSuccess) return DSW_ERR_HIP;
    if (st == 0) return DSW_OK;
    // the parity state may be half-written after a failed walk: start clean
    if (zero_workspace(s.ptr, nullptr) != DSW_OK || hipDeviceSynchronize() != hipSuccess) return DSW_ERR_HIP;
    if (st & dsw::kStatusTimeout) return DSW_ERR_DEV_TIMEOUT;
    if (st & dsw::kStatusToken) return DSW_ERR_DEV_TOKEN;
    return DSW_ERR_DEV_UNIFORMS;
}
