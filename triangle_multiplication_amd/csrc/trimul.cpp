// trimul.cpp -- host side of libtrimul: argument checks, the gfx950 gate,
// weight rounding and packing, workspace carving and the three launches.
//
// Follows the fold-cp-ops README: every data-independent decision is taken at
// construction ("Use", step 2: the constructor validates and configures,
// forward makes no decisions), and a device of the wrong architecture is
// refused up front with a message naming what was found ("Hardware" section)
// rather than failing later inside a launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "trimul.h"
#include "trimul_internal.h"
#include "trimul_launch.hpp"

struct trimul_handle {
    trimul::Params p;
    void* dev_mem;
    int device;
};

namespace {

thread_local std::string g_err;

trimul_status fail(trimul_status s, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

trimul_status ok()
{
    g_err.clear();
    return TRIMUL_OK;
}

trimul_status hip_fail(const char* what, hipError_t e)
{
    return fail(TRIMUL_ERR_HIP, "%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t elem_size(trimul_dtype t) { return t == TRIMUL_BF16 ? 2 : 4; }

bool width_ok(int x) { return x >= 32 && x <= 256 && x % 32 == 0; }

// Round to nearest even, as the hardware conversion does.
uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float bf16_to_f32(uint16_t h)
{
    const uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// Folded output GEMM for the bf16 kernels that apply LayerNorm algebraically:
// rows d of W (rows x K, fp32) become bf16(W[d][k] * gamma[k]), and each row
// gets the correction terms S_d = sum_k of the folded bf16 row and
// T_d = sum_k W[d][k] * beta[k], each split as high = bf16(v), low = bf16(v - high).
void fold_rows(const float* W, const float* gamma, const float* beta, int rows, int K,
               uint16_t* wf, uint16_t* x)
{
    for (int d = 0; d < rows; ++d) {
        double S = 0.0, T = 0.0;
        for (int k = 0; k < K; ++k) {
            const uint16_t h = f32_to_bf16((float)((double)W[(size_t)d * K + k] * gamma[k]));
            wf[(size_t)d * K + k] = h;
            S += bf16_to_f32(h);
            T += (double)W[(size_t)d * K + k] * beta[k];
        }
        const uint16_t sh = f32_to_bf16((float)S), th = f32_to_bf16((float)T);
        const uint16_t sl = f32_to_bf16((float)(S - bf16_to_f32(sh)));
        const uint16_t tl = f32_to_bf16((float)(T - bf16_to_f32(th)));
        const uint16_t row[8] = {sh, sl, sh, th, tl, th, 0, 0};
        std::memcpy(x + (size_t)d * 8, row, sizeof row);
    }
}

void put(std::vector<uint8_t>& dst, size_t off_elems, float v, trimul_dtype t)
{
    if (t == TRIMUL_BF16) {
        uint16_t h = f32_to_bf16(v);
        std::memcpy(dst.data() + off_elems * 2, &h, 2);
    } else {
        std::memcpy(dst.data() + off_elems * 4, &v, 4);
    }
}

trimul_status check_shape(const trimul_handle* h, int B, int N)
{
    if (B < 1) return fail(TRIMUL_ERR_INVALID_ARG, "B must be >= 1; got %d", B);
    if (N < 8 || N % 8 != 0)
        return fail(TRIMUL_ERR_INVALID_ARG, "N must be a multiple of 8 and >= 8 (16-byte rows); got %d", N);
    if (N > 32768) return fail(TRIMUL_ERR_UNSUPPORTED, "N must be <= 32768; got %d", N);
    if ((long long)B * h->p.C > 65535)
        return fail(TRIMUL_ERR_UNSUPPORTED, "B*C must be <= 65535; got %lld", (long long)B * h->p.C);
    // Every launch covers at most 2 threads per pair; keep that below 2^32.
    if ((long long)B * N * N >= (1LL << 31))
        return fail(TRIMUL_ERR_UNSUPPORTED, "B*N*N must be < 2^31; got %lld", (long long)B * N * N);
    return TRIMUL_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    if (!a || !b || !na || !nb) return false;
    uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

trimul_status check_handle_device(const trimul_handle* h)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev != h->device)
        return fail(TRIMUL_ERR_INVALID_ARG, "handle was created on device %d but device %d is current",
                    h->device, dev);
    return TRIMUL_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

const char* trimul_status_string(trimul_status s)
{
    switch (s) {
    case TRIMUL_OK: return "TRIMUL_OK";
    case TRIMUL_ERR_INVALID_ARG: return "TRIMUL_ERR_INVALID_ARG";
    case TRIMUL_ERR_UNSUPPORTED: return "TRIMUL_ERR_UNSUPPORTED";
    case TRIMUL_ERR_ARCH: return "TRIMUL_ERR_ARCH";
    case TRIMUL_ERR_WORKSPACE: return "TRIMUL_ERR_WORKSPACE";
    case TRIMUL_ERR_HIP: return "TRIMUL_ERR_HIP";
    }
    return "TRIMUL_ERR_UNKNOWN";
}

const char* trimul_last_error(void) { return g_err.c_str(); }

trimul_status trimul_check_arch(const char* name)
{
    if (!name) return fail(TRIMUL_ERR_INVALID_ARG, "architecture name is NULL");
    if (std::strncmp(name, "gfx950", 6) == 0 && (name[6] == '\0' || name[6] == ':')) return ok();
    return fail(TRIMUL_ERR_ARCH, "libtrimul requires gfx950 (MI355X); got %s", name);
}

trimul_status trimul_workspace_query(int D, int C, trimul_dtype dtype, int B, int N, size_t* bytes)
{
    if (!bytes) return fail(TRIMUL_ERR_INVALID_ARG, "bytes is NULL");
    if (dtype != TRIMUL_BF16 && dtype != TRIMUL_FP32)
        return fail(TRIMUL_ERR_INVALID_ARG, "dtype must be TRIMUL_BF16 or TRIMUL_FP32; got %d", (int)dtype);
    if (!width_ok(D) || !width_ok(C))
        return fail(TRIMUL_ERR_UNSUPPORTED, "D and C must be multiples of 32 in [32, 256]; got D=%d C=%d", D, C);
    if (B < 1 || N < 1) return fail(TRIMUL_ERR_INVALID_ARG, "B and N must be >= 1; got B=%d N=%d", B, N);
    const trimul::DType t = dtype == TRIMUL_BF16 ? trimul::DType::BF16 : trimul::DType::FP32;
    const size_t ab = align256((size_t)B * C * trimul::ab_slab_elems(t, N) * elem_size(dtype));
    const size_t o = align256((size_t)B * C * (size_t)N * N * elem_size(dtype));
    *bytes = 2 * ab + o;
    return ok();
}

trimul_status trimul_workspace_size(const trimul_handle* h, int B, int N, size_t* bytes)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    return trimul_workspace_query(h->p.D, h->p.C, (trimul_dtype)h->p.dtype, B, N, bytes);
}

trimul_status trimul_create(int D, int C, trimul_dtype dtype, const trimul_weights* w,
                            trimul_handle** out)
{
    if (!out) return fail(TRIMUL_ERR_INVALID_ARG, "out (handle pointer) is NULL");
    *out = nullptr;
    if (!w) return fail(TRIMUL_ERR_INVALID_ARG, "weights is NULL");
    if (dtype != TRIMUL_BF16 && dtype != TRIMUL_FP32)
        return fail(TRIMUL_ERR_INVALID_ARG, "dtype must be TRIMUL_BF16 or TRIMUL_FP32; got %d", (int)dtype);
    if (!width_ok(D) || !width_ok(C))
        return fail(TRIMUL_ERR_UNSUPPORTED, "D and C must be multiples of 32 in [32, 256]; got D=%d C=%d", D, C);
    const struct { const float* p; const char* n; } req[] = {
        {w->norm_in_weight, "norm_in_weight"}, {w->norm_in_bias, "norm_in_bias"},
        {w->p_in, "p_in"}, {w->g_in, "g_in"}, {w->norm_out_weight, "norm_out_weight"},
        {w->norm_out_bias, "norm_out_bias"}, {w->p_out, "p_out"}, {w->g_out, "g_out"}};
    for (const auto& r : req)
        if (!r.p) return fail(TRIMUL_ERR_INVALID_ARG, "weights->%s is NULL", r.n);
    if (!(w->eps > 0.0f) || !std::isfinite(w->eps))
        return fail(TRIMUL_ERR_INVALID_ARG, "eps must be finite and > 0; got %g", (double)w->eps);

    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail("hipGetDeviceProperties", e);
    trimul_status st = trimul_check_arch(prop.gcnArchName);
    if (st != TRIMUL_OK) return st;

    // Host packing.
    const size_t es = elem_size(dtype);
    const size_t n_proj = (size_t)4 * C * D, n_go = (size_t)D * D, n_po = (size_t)D * C;
    const size_t off_proj = 0;
    const size_t off_go = align256(n_proj * es);
    const size_t off_po = off_go + align256(n_go * es);
    const size_t off_ln = off_po + align256(n_po * es);
    const size_t off_gof = off_ln + align256((size_t)(2 * D + 2 * C) * 4);
    const bool folded = dtype == TRIMUL_BF16;
    const size_t off_pof = off_gof + (folded ? align256(n_go * 2) : 0);
    const size_t off_xg = off_pof + (folded ? align256(n_po * 2) : 0);
    const size_t off_xp = off_xg + (folded ? align256((size_t)D * 16) : 0);
    const size_t off_wpf = off_xp + (folded ? align256((size_t)D * 16) : 0);
    const size_t off_xpj = off_wpf + (folded ? align256(n_proj * 2) : 0);
    const size_t off_sink = off_xpj + (folded ? align256((size_t)4 * C * 16) : 0);
    const size_t total = off_sink + 4096;
    std::vector<uint8_t> host(total, 0);
    if (folded) {
        fold_rows(w->g_out, w->norm_in_weight, w->norm_in_bias, D, D,
                  reinterpret_cast<uint16_t*>(host.data() + off_gof),
                  reinterpret_cast<uint16_t*>(host.data() + off_xg));
        fold_rows(w->p_out, w->norm_out_weight, w->norm_out_bias, D, C,
                  reinterpret_cast<uint16_t*>(host.data() + off_pof),
                  reinterpret_cast<uint16_t*>(host.data() + off_xp));
    }
    {
        std::vector<uint8_t> go(n_go * es), po(n_po * es);
        // Projection rows in the kernels' order: for a then b, per 16-channel
        // group, 16 rows of p_in then the same channels' 16 rows of g_in.
        std::vector<float> projf(n_proj);
        size_t row = 0;
        for (int part = 0; part < 2; ++part)          // a, then b
            for (int g = 0; g < C / 16; ++g) {        // 16-channel groups
                for (int r = 0; r < 16; ++r, ++row)   // p rows
                    std::memcpy(&projf[row * D], w->p_in + ((size_t)part * C + g * 16 + r) * D, D * 4);
                for (int r = 0; r < 16; ++r, ++row)   // g rows of the same channels
                    std::memcpy(&projf[row * D], w->g_in + ((size_t)part * C + g * 16 + r) * D, D * 4);
            }
        std::vector<uint8_t> proj(n_proj * es);
        for (size_t i = 0; i < n_proj; ++i) put(proj, i, projf[i], dtype);
        if (folded)
            fold_rows(projf.data(), w->norm_in_weight, w->norm_in_bias, 4 * C, D,
                      reinterpret_cast<uint16_t*>(host.data() + off_wpf),
                      reinterpret_cast<uint16_t*>(host.data() + off_xpj));
        for (size_t i = 0; i < n_go; ++i) put(go, i, w->g_out[i], dtype);
        for (size_t i = 0; i < n_po; ++i) put(po, i, w->p_out[i], dtype);
        std::memcpy(host.data() + off_proj, proj.data(), proj.size());
        std::memcpy(host.data() + off_go, go.data(), go.size());
        std::memcpy(host.data() + off_po, po.data(), po.size());
        float* ln = reinterpret_cast<float*>(host.data() + off_ln);
        std::memcpy(ln, w->norm_in_weight, D * 4);
        std::memcpy(ln + D, w->norm_in_bias, D * 4);
        std::memcpy(ln + 2 * D, w->norm_out_weight, C * 4);
        std::memcpy(ln + 2 * D + C, w->norm_out_bias, C * 4);
    }

    void* mem = nullptr;
    e = hipMalloc(&mem, total);
    if (e != hipSuccess) return hip_fail("hipMalloc (packed weights)", e);
    e = hipMemcpy(mem, host.data(), total, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(mem);
        return hip_fail("hipMemcpy (packed weights)", e);
    }
    trimul_handle* h = new (std::nothrow) trimul_handle;
    if (!h) {
        (void)hipFree(mem);
        return fail(TRIMUL_ERR_INVALID_ARG, "out of host memory");
    }
    uint8_t* base = static_cast<uint8_t*>(mem);
    h->dev_mem = mem;
    h->device = dev;
    h->p.D = D;
    h->p.C = C;
    h->p.dtype = dtype == TRIMUL_BF16 ? trimul::DType::BF16 : trimul::DType::FP32;
    h->p.eps = w->eps;
    h->p.w_proj = base + off_proj;
    h->p.w_gout = base + off_go;
    h->p.w_pout = base + off_po;
    const float* ln = reinterpret_cast<const float*>(base + off_ln);
    h->p.ln_in_w = ln;
    h->p.ln_in_b = ln + D;
    h->p.ln_out_w = ln + 2 * D;
    h->p.ln_out_b = ln + 2 * D + C;
    h->p.w_gout_f = folded ? base + off_gof : nullptr;
    h->p.w_pout_f = folded ? base + off_pof : nullptr;
    h->p.x_gout = folded ? base + off_xg : nullptr;
    h->p.x_pout = folded ? base + off_xp : nullptr;
    h->p.w_proj_f = folded ? base + off_wpf : nullptr;
    h->p.x_proj = folded ? base + off_xpj : nullptr;
    h->p.sink = base + off_sink;
    *out = h;
    return ok();
}

void trimul_destroy(trimul_handle* h)
{
    if (!h) return;
    if (h->dev_mem) (void)hipFree(h->dev_mem);
    delete h;
}

trimul_status trimul_fwd(trimul_handle* h, const void* z, const void* pair_mask, int B, int N,
                         trimul_direction dir, void* out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    if (!z) return fail(TRIMUL_ERR_INVALID_ARG, "z is NULL");
    if (!out) return fail(TRIMUL_ERR_INVALID_ARG, "out is NULL");
    if (dir != TRIMUL_OUTGOING && dir != TRIMUL_INCOMING)
        return fail(TRIMUL_ERR_INVALID_ARG, "direction must be TRIMUL_OUTGOING or TRIMUL_INCOMING; got %d", (int)dir);
    trimul_status st = check_shape(h, B, N);
    if (st != TRIMUL_OK) return st;
    const trimul_dtype dt = (trimul_dtype)h->p.dtype;
    const size_t es = elem_size(dt);
    if (!aligned(z, 16)) return fail(TRIMUL_ERR_INVALID_ARG, "z must be 16-byte aligned");
    if (!aligned(out, 16)) return fail(TRIMUL_ERR_INVALID_ARG, "out must be 16-byte aligned");
    if (pair_mask && !aligned(pair_mask, es))
        return fail(TRIMUL_ERR_INVALID_ARG, "pair_mask must be aligned to its element size");
    size_t need = 0;
    st = trimul_workspace_query(h->p.D, h->p.C, dt, B, N, &need);
    if (st != TRIMUL_OK) return st;
    if (!workspace) return fail(TRIMUL_ERR_WORKSPACE, "workspace is NULL (%zu bytes required)", need);
    if (workspace_bytes < need)
        return fail(TRIMUL_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                    workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(TRIMUL_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const size_t NN = (size_t)N * N;
    const size_t zbytes = (size_t)B * NN * h->p.D * es;
    const size_t mbytes = pair_mask ? (size_t)B * NN * es : 0;
    if (overlaps(out, zbytes, z, zbytes)) return fail(TRIMUL_ERR_INVALID_ARG, "out overlaps z");
    if (overlaps(out, zbytes, pair_mask, mbytes)) return fail(TRIMUL_ERR_INVALID_ARG, "out overlaps pair_mask");
    if (overlaps(out, zbytes, workspace, need)) return fail(TRIMUL_ERR_INVALID_ARG, "out overlaps the workspace");
    if (overlaps(z, zbytes, workspace, need)) return fail(TRIMUL_ERR_INVALID_ARG, "z overlaps the workspace");
    if (overlaps(pair_mask, mbytes, workspace, need))
        return fail(TRIMUL_ERR_INVALID_ARG, "pair_mask overlaps the workspace");
    st = check_handle_device(h);
    if (st != TRIMUL_OK) return st;

    const size_t ab = align256((size_t)B * h->p.C * trimul::ab_slab_elems(h->p.dtype, N) * es);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    void* a = ws;
    void* b = ws + ab;
    void* o = ws + 2 * ab;
    hipError_t e = trimul::launch_project(h->p, z, pair_mask, B, N, dir == TRIMUL_INCOMING, a, b, stream);
    if (e != hipSuccess) return hip_fail("projection kernel launch", e);
    e = trimul::launch_contract(h->p, a, b, B, N, o, stream);
    if (e != hipSuccess) return hip_fail("contraction kernel launch", e);
    e = trimul::launch_output(h->p, z, o, B, N, out, stream);
    if (e != hipSuccess) return hip_fail("output kernel launch", e);
    return ok();
}

trimul_status trimul_internal_project(trimul_handle* h, const void* z, const void* pair_mask, int B,
                                      int N, trimul_direction dir, void* a_cm, void* b_cm,
                                      hipStream_t stream)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    if (!z || !a_cm || !b_cm) return fail(TRIMUL_ERR_INVALID_ARG, "z, a_cm and b_cm must be non-NULL");
    if (dir != TRIMUL_OUTGOING && dir != TRIMUL_INCOMING)
        return fail(TRIMUL_ERR_INVALID_ARG, "direction must be TRIMUL_OUTGOING or TRIMUL_INCOMING; got %d", (int)dir);
    trimul_status st = check_shape(h, B, N);
    if (st != TRIMUL_OK) return st;
    if (!aligned(z, 16) || !aligned(a_cm, 16) || !aligned(b_cm, 16))
        return fail(TRIMUL_ERR_INVALID_ARG, "z, a_cm and b_cm must be 16-byte aligned");
    st = check_handle_device(h);
    if (st != TRIMUL_OK) return st;
    hipError_t e = trimul::launch_project(h->p, z, pair_mask, B, N, dir == TRIMUL_INCOMING, a_cm, b_cm, stream);
    if (e != hipSuccess) return hip_fail("projection kernel launch", e);
    return ok();
}

trimul_status trimul_internal_contract(trimul_handle* h, const void* a_cm, const void* b_cm, int B,
                                       int N, void* o, hipStream_t stream)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    if (!a_cm || !b_cm || !o) return fail(TRIMUL_ERR_INVALID_ARG, "a_cm, b_cm and o must be non-NULL");
    trimul_status st = check_shape(h, B, N);
    if (st != TRIMUL_OK) return st;
    if (!aligned(a_cm, 16) || !aligned(b_cm, 16) || !aligned(o, 16))
        return fail(TRIMUL_ERR_INVALID_ARG, "a_cm, b_cm and o must be 16-byte aligned");
    st = check_handle_device(h);
    if (st != TRIMUL_OK) return st;
    hipError_t e = trimul::launch_contract(h->p, a_cm, b_cm, B, N, o, stream);
    if (e != hipSuccess) return hip_fail("contraction kernel launch", e);
    return ok();
}

trimul_status trimul_internal_output(trimul_handle* h, const void* z, const void* o, int B, int N,
                                     void* out, hipStream_t stream)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    if (!z || !o || !out) return fail(TRIMUL_ERR_INVALID_ARG, "z, o and out must be non-NULL");
    trimul_status st = check_shape(h, B, N);
    if (st != TRIMUL_OK) return st;
    if (!aligned(z, 16) || !aligned(o, 16) || !aligned(out, 16))
        return fail(TRIMUL_ERR_INVALID_ARG, "z, o and out must be 16-byte aligned");
    st = check_handle_device(h);
    if (st != TRIMUL_OK) return st;
    hipError_t e = trimul::launch_output(h->p, z, o, B, N, out, stream);
    if (e != hipSuccess) return hip_fail("output kernel launch", e);
    return ok();
}

}  // extern "C"
