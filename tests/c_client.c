/*
 * c_client.c -- a plain C program that drives libdeltalog through its C ABI
 * (include/deltalog.h) with device memory from the HIP runtime: no Python, no
 * torch.  Test infrastructure: tests/test_c_client_gpu.py writes the inputs,
 * runs this program on the GPU and checks its outputs against the oracle.
 *
 *   c_client IN OUT
 *
 * IN (little-endian): int32 op, B, H, dk, dv, M, T; then float32 arrays
 * base [B,H,dk,dv], u [H,dk] (RWKV6 only), and for each of the T steps
 * q [B,H,dk], k [B,H,dk], v [B,H,dv], beta [B,H] (not for RWKV6),
 * log-decay [B,H] (GDN) or [B,H,dk].  Inputs are fp32.
 * OUT: float32 o [T,B,H,dv], then the base [B,H,dk,dv] after a final
 * dl_merge.  Exit status 0 on success; otherwise the failing call is printed.
 */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "deltalog.h"

static int fail(const char *what, int code)
{
    fprintf(stderr, "c_client: %s failed (%d)\n", what, code);
    return 1;
}

static float *read_floats(FILE *f, size_t n)
{
    float *p = (float *)malloc(n * sizeof(float));
    if (p && fread(p, sizeof(float), n, f) != n) {
        free(p);
        return NULL;
    }
    return p;
}

static void *to_device(const float *h, size_t n)
{
    void *d = NULL;
    if (hipMalloc(&d, n * sizeof(float)) != hipSuccess)
        return NULL;
    if (hipMemcpy(d, h, n * sizeof(float), hipMemcpyHostToDevice) != hipSuccess)
        return NULL;
    return d;
}

int main(int argc, char **argv)
{
    if (argc != 3)
        return fail("usage: c_client IN OUT", 2);
    FILE *in = fopen(argv[1], "rb");
    if (!in)
        return fail("open IN", 2);
    int hdr[7];
    if (fread(hdr, sizeof(int), 7, in) != 7)
        return fail("read header", 2);
    const int op = hdr[0], B = hdr[1], H = hdr[2], dk = hdr[3], dv = hdr[4], M = hdr[5], T = hdr[6];
    const size_t BH = (size_t)B * H, P = BH * dk * dv;
    const size_t nld = op == DL_OP_GDN ? BH : BH * dk;

    float *h_base = read_floats(in, P);
    float *h_u = op == DL_OP_RWKV6 ? read_floats(in, (size_t)H * dk) : NULL;
    if (!h_base || (op == DL_OP_RWKV6 && !h_u))
        return fail("read base/u", 2);
    void *d_base = to_device(h_base, P);
    void *d_u = h_u ? to_device(h_u, (size_t)H * dk) : NULL;

    const size_t ws_bytes = dl_workspace_bytes(B, H, dk, dv, M, (dl_op)op, DL_F32);
    if (ws_bytes == 0)
        return fail("dl_workspace_bytes", 0);
    void *d_ws = NULL;
    if (!d_base || hipMalloc(&d_ws, ws_bytes) != hipSuccess)
        return fail("hipMalloc", 0);

    dl_state *s = NULL;
    dl_status st = dl_state_create(B, H, dk, dv, M, (dl_op)op, DL_F32, (float *)d_base, d_ws,
                                   (const float *)d_u, &s);
    if (st != DL_OK)
        return fail(dl_status_string(st), st);

    hipStream_t stream;
    if (hipStreamCreate(&stream) != hipSuccess)
        return fail("hipStreamCreate", 0);
    float *h_o = (float *)malloc((size_t)T * BH * dv * sizeof(float));
    void *d_o = NULL;
    if (!h_o || hipMalloc(&d_o, BH * dv * sizeof(float)) != hipSuccess)
        return fail("alloc o", 0);

    for (int t = 0; t < T; ++t) {
        float *q = read_floats(in, BH * dk), *k = read_floats(in, BH * dk), *v = read_floats(in, BH * dv);
        float *beta = op == DL_OP_RWKV6 ? NULL : read_floats(in, BH);
        float *ld = read_floats(in, nld);
        if (!q || !k || !v || (op != DL_OP_RWKV6 && !beta) || !ld)
            return fail("read step", 2);
        void *dq = to_device(q, BH * dk), *dk_ = to_device(k, BH * dk), *dvv = to_device(v, BH * dv);
        void *dbeta = beta ? to_device(beta, BH) : NULL, *dld = to_device(ld, nld);
        st = dl_decode_step(s, dq, dk_, dvv, (const float *)dbeta, (const float *)dld, (float *)d_o,
                            (void *)stream);
        if (st != DL_OK)
            return fail(dl_status_string(st), st);
        if (hipMemcpyAsync(h_o + (size_t)t * BH * dv, d_o, BH * dv * sizeof(float), hipMemcpyDeviceToHost,
                           stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess)
            return fail("copy o", 0);
        hipFree(dq);
        hipFree(dk_);
        hipFree(dvv);
        if (dbeta)
            hipFree(dbeta);
        hipFree(dld);
        free(q);
        free(k);
        free(v);
        free(beta);
        free(ld);
    }
    st = dl_merge(s, (void *)stream);
    if (st != DL_OK)
        return fail(dl_status_string(st), st);
    if (hipMemcpyAsync(h_base, d_base, P * sizeof(float), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return fail("copy base", 0);
    fclose(in);

    FILE *out = fopen(argv[2], "wb");
    if (!out || fwrite(h_o, sizeof(float), (size_t)T * BH * dv, out) != (size_t)T * BH * dv ||
        fwrite(h_base, sizeof(float), P, out) != P)
        return fail("write OUT", 2);
    fclose(out);

    dl_state_destroy(s);
    hipStreamDestroy(stream);
    hipFree(d_o);
    hipFree(d_ws);
    hipFree(d_base);
    if (d_u)
        hipFree(d_u);
    free(h_o);
    free(h_base);
    free(h_u);
    return 0;
}
