/*
 * A C11 program that uses libcpattn through include/cpattn.h alone: device
 * memory and the stream come from the HIP runtime's C API, nothing from
 * PyTorch or Python.  It runs one small instance of the per-rank path and
 * writes the results for the caller to check against the oracle:
 *
 *   1. attention over all keys, bf16 in / bf16 out          -> O, LSE
 *   2. attention over keys [0, Skv_a) and [Skv_a, Skv) with f32 outputs,
 *      then attn_merge of the two partials (Ring Attention's blockwise
 *      combination of partial results)                     -> O, LSE (f32)
 *   3. Ulysses pack (sequence -> head) of q's words read as a
 *      [B, S_local, H, D] shard, then the inverse unpack (head -> sequence)
 *                                                          -> packed buffer;
 *      the round trip is checked bit for bit here
 *
 * Usage: c_consumer IN OUT.  IN holds six int64 (B, H, S, Skv, D, Skv_a) and
 * one double (the score scale), then q [B,H,S,D], k and v [B,H,Skv,D] as raw
 * bf16 words; OUT
 * receives O bf16, LSE f32, merged O f32, merged LSE f32 and the packed
 * buffer (bf16 words), in that order.  Any failed call prints its status
 * and the program exits non-zero.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "cpattn.h"

#define HIP_OK(x)                                                                    \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x,              \
                    hipGetErrorString(e_));                                          \
            exit(2);                                                                 \
        }                                                                            \
    } while (0)

#define CP_OK(x)                                                                     \
    do {                                                                             \
        cpattn_status s_ = (x);                                                      \
        if (s_ != CPATTN_OK) {                                                       \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x,              \
                    cpattn_status_string(s_));                                       \
            exit(3);                                                                 \
        }                                                                            \
    } while (0)

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    HIP_OK(hipMalloc(&p, bytes ? bytes : 16));
    return p;
}

static void* read_exact(FILE* f, size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p || fread(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "short input\n");
        exit(4);
    }
    return p;
}

static void write_back(FILE* f, const void* dev, size_t bytes) {
    void* h = malloc(bytes ? bytes : 1);
    if (!h) exit(5);
    HIP_OK(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
    if (fwrite(h, 1, bytes, f) != bytes) exit(5);
    free(h);
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
        return 1;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in) return 1;
    int64_t hdr[6];
    double scale_in;
    if (fread(hdr, sizeof hdr, 1, in) != 1 || fread(&scale_in, sizeof scale_in, 1, in) != 1) return 4;
    const int64_t B = hdr[0], H = hdr[1], S = hdr[2], Skv = hdr[3], D = hdr[4], Skv_a = hdr[5];
    const int64_t P = H;   /* relayout ranks: one head each after the exchange */
    if (B < 1 || H < 1 || S < 1 || Skv_a < 1 || Skv_a >= Skv || (D != 64 && D != 128)) return 1;
    const size_t q_elems = (size_t)(B * H * S * D), kv_elems = (size_t)(B * H * Skv * D);
    const size_t rows = (size_t)(B * H * S);
    void* hq = read_exact(in, q_elems * 2);
    void* hk = read_exact(in, kv_elems * 2);
    void* hv = read_exact(in, kv_elems * 2);
    fclose(in);

    printf("cpattn ABI %d: B=%lld H=%lld S=%lld Skv=%lld D=%lld split at %lld\n", CPATTN_ABI_VERSION,
           (long long)B, (long long)H, (long long)S, (long long)Skv, (long long)D, (long long)Skv_a);
    fflush(stdout);

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    uint16_t *q = dev_alloc(q_elems * 2), *k = dev_alloc(kv_elems * 2), *v = dev_alloc(kv_elems * 2);
    HIP_OK(hipMemcpy(q, hq, q_elems * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(k, hk, kv_elems * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v, hv, kv_elems * 2, hipMemcpyHostToDevice));

    /* 1. all keys, bf16 output */
    uint16_t* o = dev_alloc(q_elems * 2);
    float* lse = dev_alloc(rows * 4);
    const float scale = (float)scale_in;
    CP_OK(cpattn_attn_fwd(q, k, v, o, lse, B, H, S, Skv, D, scale, CPATTN_BF16, CPATTN_BF16, stream));

    /* 2. the two key ranges as separate calls (each head's keys are split, so the
     * ranges are copied out per (b, h) into their own [B, H, Skv_x, D] tensors) */
    const int64_t Skv_b = Skv - Skv_a;
    uint16_t *ka = dev_alloc((size_t)(B * H * Skv_a * D) * 2), *va = dev_alloc((size_t)(B * H * Skv_a * D) * 2);
    uint16_t *kb = dev_alloc((size_t)(B * H * Skv_b * D) * 2), *vb = dev_alloc((size_t)(B * H * Skv_b * D) * 2);
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const size_t src = (size_t)(bh * Skv * D), na = (size_t)(Skv_a * D), nb = (size_t)(Skv_b * D);
        HIP_OK(hipMemcpyAsync(ka + bh * na, k + src, na * 2, hipMemcpyDeviceToDevice, stream));
        HIP_OK(hipMemcpyAsync(va + bh * na, v + src, na * 2, hipMemcpyDeviceToDevice, stream));
        HIP_OK(hipMemcpyAsync(kb + bh * nb, k + src + na, nb * 2, hipMemcpyDeviceToDevice, stream));
        HIP_OK(hipMemcpyAsync(vb + bh * nb, v + src + na, nb * 2, hipMemcpyDeviceToDevice, stream));
    }
    float *oa = dev_alloc(q_elems * 4), *ob = dev_alloc(q_elems * 4);
    float *la = dev_alloc(rows * 4), *lb = dev_alloc(rows * 4);
    CP_OK(cpattn_attn_fwd(q, ka, va, oa, la, B, H, S, Skv_a, D, scale, CPATTN_BF16, CPATTN_F32, stream));
    CP_OK(cpattn_attn_fwd(q, kb, vb, ob, lb, B, H, S, Skv_b, D, scale, CPATTN_BF16, CPATTN_F32, stream));
    CP_OK(cpattn_attn_merge(oa, la, ob, lb, oa, la, B, H, S, D, CPATTN_F32, stream));   /* in place */

    /* 3. Ulysses relayout: q's words read as one rank's [B, S_local = S, H, D] shard,
     * exchanged over P = H ranks (one head each) */
    uint16_t* packed = dev_alloc(q_elems * 2);
    uint16_t* back = dev_alloc(q_elems * 2);
    CP_OK(cpattn_ulysses_pack(q, packed, B, S, H, D, P, CPATTN_BF16, CPATTN_SEQ_TO_HEAD, stream));
    CP_OK(cpattn_ulysses_unpack(packed, back, B, S, H, D, P, CPATTN_BF16, CPATTN_HEAD_TO_SEQ, stream));
    HIP_OK(hipStreamSynchronize(stream));

    void* hback = malloc(q_elems * 2);
    if (!hback) return 5;
    HIP_OK(hipMemcpy(hback, back, q_elems * 2, hipMemcpyDeviceToHost));
    if (memcmp(hback, hq, q_elems * 2) != 0) {
        fprintf(stderr, "pack/unpack round trip is not the identity\n");
        return 6;
    }

    FILE* out = fopen(argv[2], "wb");
    if (!out) return 1;
    write_back(out, o, q_elems * 2);
    write_back(out, lse, rows * 4);
    write_back(out, oa, q_elems * 4);
    write_back(out, la, rows * 4);
    write_back(out, packed, q_elems * 2);
    fclose(out);

    void* bufs[] = {q, k, v, o, lse, ka, va, kb, vb, oa, ob, la, lb, packed, back};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
    HIP_OK(hipStreamDestroy(stream));
    free(hq);
    free(hk);
    free(hv);
    free(hback);
    printf("ok\n");
    return 0;
}
