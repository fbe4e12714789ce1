/*
 * A plain C caller of libltree, with no Python and no torch: it reads one
 * tree-verification problem from a binary file, runs ltree_build_mask and
 * ltree_attn through the C ABI on device buffers from hipMalloc, then the
 * same problem through ltree_attn_noalloc and through ltree_attn_strided over
 * an interleaved copy of the prefix cache [total_L, 2, Hkv, D], and writes the
 * mask and the three (o, lse) results to an output file.  The GPU test that
 * drives it checks them against the fp64 oracle and against each other.
 *
 * Input (little-endian): int32 B, T, Hq, Hkv, D, dtype (ltree_dtype),
 * max_prefix_len, total_L; float32 scale; int32 parent[B*T];
 * int32 offsets[B+1]; then q [B,T,Hq,D], k_prefix and v_prefix
 * [total_L,Hkv,D], k_tree and v_tree [B,T,Hkv,D], each in the element type
 * (2 bytes for bf16, 4 for fp32).
 * Output: int32 library status of each call (mask, attn, noalloc, strided),
 * int32 mask status word, uint64 mask[B*T*W], then for attn, noalloc and
 * strided in turn float32 o[B*T*Hq*D] and float32 lse[B*Hq*T].
 *
 *   ltree_c_caller <input> <output>      exit code 0 when every step ran
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ltree.h"

static int fail(const char* what) {
  fprintf(stderr, "ltree_c_caller: %s\n", what);
  return 1;
}

static void* read_block(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p != NULL && bytes > 0 && fread(p, 1, bytes, f) != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 16) != hipSuccess) return NULL;
  if (bytes > 0 && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) return fail("usage: ltree_c_caller <input> <output>");
  FILE* in = fopen(argv[1], "rb");
  if (in == NULL) return fail("cannot open the input");
  int32_t h[8];
  float scale;
  if (fread(h, sizeof(h), 1, in) != 1 || fread(&scale, sizeof(scale), 1, in) != 1) {
    return fail("short header");
  }
  const int B = h[0], T = h[1], Hq = h[2], Hkv = h[3], D = h[4], max_len = h[6], total = h[7];
  const ltree_dtype dtype = (ltree_dtype)h[5];
  const size_t e = dtype == LTREE_BF16 ? 2 : 4;
  const size_t W = LTREE_MASK_WORDS(T);
  const size_t nq = (size_t)B * T * Hq * D, nkp = (size_t)total * Hkv * D;
  const size_t nkt = (size_t)B * T * Hkv * D;
  void* parent = read_block(in, sizeof(int32_t) * B * T);
  void* offsets = read_block(in, sizeof(int32_t) * (B + 1));
  void* q = read_block(in, nq * e);
  void* kp = read_block(in, nkp * e);
  void* vp = read_block(in, nkp * e);
  void* kt = read_block(in, nkt * e);
  void* vt = read_block(in, nkt * e);
  fclose(in);
  if (!parent || !offsets || !q || !kp || !vp || !kt || !vt) return fail("short input");

  void* d_parent = to_device(parent, sizeof(int32_t) * B * T);
  void* d_off = to_device(offsets, sizeof(int32_t) * (B + 1));
  void* d_q = to_device(q, nq * e);
  void* d_kp = to_device(kp, nkp * e);
  void* d_vp = to_device(vp, nkp * e);
  void* d_kt = to_device(kt, nkt * e);
  void* d_vt = to_device(vt, nkt * e);
  /* the prefix cache interleaved: row t holds K then V of all KV heads */
  const size_t row_bytes = (size_t)Hkv * D * e;
  char* kv = (char*)malloc(2 * row_bytes * (total ? total : 1));
  if (kv == NULL) return fail("malloc failed");
  for (size_t t = 0; t < (size_t)total; ++t) {
    const char* ks = (const char*)kp + t * row_bytes;
    const char* vs = (const char*)vp + t * row_bytes;
    for (size_t i = 0; i < row_bytes; ++i) {
      kv[2 * t * row_bytes + i] = ks[i];
      kv[(2 * t + 1) * row_bytes + i] = vs[i];
    }
  }
  void* d_kv = to_device(kv, 2 * row_bytes * total);
  const int64_t kv_stride = 2 * (int64_t)Hkv * D;
  void *d_mask = NULL, *d_status = NULL, *d_o = NULL, *d_lse = NULL, *d_ws = NULL;
  void *d_o2 = NULL, *d_lse2 = NULL, *d_o3 = NULL, *d_lse3 = NULL, *d_ws3 = NULL;
  const size_t ws_bytes = ltree_attn_workspace_bytes(B, T, Hq, Hkv, D, max_len);
  const size_t ws3_bytes =
      ltree_attn_strided_workspace_bytes(B, T, Hq, Hkv, D, max_len, kv_stride, kv_stride);
  if (ws_bytes == 0 || ws3_bytes == 0) return fail("invalid sizes");
  if (hipMalloc(&d_mask, sizeof(uint64_t) * B * T * W) != hipSuccess ||
      hipMalloc(&d_status, sizeof(int32_t)) != hipSuccess ||
      hipMalloc(&d_o, sizeof(float) * nq) != hipSuccess ||
      hipMalloc(&d_lse, sizeof(float) * B * Hq * T) != hipSuccess ||
      hipMalloc(&d_ws, ws_bytes) != hipSuccess || hipMalloc(&d_o2, sizeof(float) * nq) != hipSuccess ||
      hipMalloc(&d_lse2, sizeof(float) * B * Hq * T) != hipSuccess ||
      hipMalloc(&d_o3, sizeof(float) * nq) != hipSuccess ||
      hipMalloc(&d_lse3, sizeof(float) * B * Hq * T) != hipSuccess ||
      hipMalloc(&d_ws3, ws3_bytes) != hipSuccess) {
    return fail("hipMalloc failed");
  }
  if (!d_parent || !d_off || !d_q || !d_kp || !d_vp || !d_kt || !d_vt || !d_kv) {
    return fail("upload failed");
  }

  hipStream_t stream;
  if (hipStreamCreate(&stream) != hipSuccess) return fail("hipStreamCreate failed");
  int32_t rc[4];
  rc[0] = ltree_build_mask((const int32_t*)d_parent, B, T, (uint64_t*)d_mask, (int32_t*)d_status,
                           stream);
  rc[1] = ltree_attn(dtype, B, T, Hq, Hkv, D, scale, d_q, d_kp, d_vp, (const int32_t*)d_off,
                     max_len, d_kt, d_vt, (const uint64_t*)d_mask, (float*)d_o, (float*)d_lse,
                     d_ws, ws_bytes, stream);
  rc[2] = ltree_attn_noalloc(dtype, B, T, Hq, Hkv, D, scale, d_q, d_kp, d_vp,
                             (const int32_t*)d_off, max_len, d_kt, d_vt, (const uint64_t*)d_mask,
                             (float*)d_o2, (float*)d_lse2, stream);
  rc[3] = ltree_attn_strided(dtype, B, T, Hq, Hkv, D, scale, d_q, d_kv, (char*)d_kv + row_bytes,
                             kv_stride, kv_stride, (const int32_t*)d_off, max_len, d_kt, d_vt,
                             (const uint64_t*)d_mask, (float*)d_o3, (float*)d_lse3, d_ws3,
                             ws3_bytes, stream);
  if (hipStreamSynchronize(stream) != hipSuccess) return fail("stream failed");
  printf("ltree %d: build_mask %s, attn %s, noalloc %s, strided %s\n", ltree_version(),
         ltree_status_string(rc[0]), ltree_status_string(rc[1]), ltree_status_string(rc[2]),
         ltree_status_string(rc[3]));

  int32_t status = -1;
  uint64_t* mask = (uint64_t*)malloc(sizeof(uint64_t) * B * T * W);
  float* o = (float*)malloc(sizeof(float) * nq);
  float* lse = (float*)malloc(sizeof(float) * B * Hq * T);
  float* o2 = (float*)malloc(sizeof(float) * nq);
  float* lse2 = (float*)malloc(sizeof(float) * B * Hq * T);
  float* o3 = (float*)malloc(sizeof(float) * nq);
  float* lse3 = (float*)malloc(sizeof(float) * B * Hq * T);
  if (!mask || !o || !lse || !o2 || !lse2 || !o3 || !lse3) return fail("malloc failed");
  if (hipMemcpy(&status, d_status, sizeof(status), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(mask, d_mask, sizeof(uint64_t) * B * T * W, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(o, d_o, sizeof(float) * nq, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(lse, d_lse, sizeof(float) * B * Hq * T, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(o2, d_o2, sizeof(float) * nq, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(lse2, d_lse2, sizeof(float) * B * Hq * T, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(o3, d_o3, sizeof(float) * nq, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(lse3, d_lse3, sizeof(float) * B * Hq * T, hipMemcpyDeviceToHost) != hipSuccess) {
    return fail("download failed");
  }
  FILE* out = fopen(argv[2], "wb");
  if (out == NULL) return fail("cannot open the output");
  fwrite(rc, sizeof(rc), 1, out);
  fwrite(&status, sizeof(status), 1, out);
  fwrite(mask, sizeof(uint64_t), (size_t)B * T * W, out);
  fwrite(o, sizeof(float), nq, out);
  fwrite(lse, sizeof(float), (size_t)B * Hq * T, out);
  fwrite(o2, sizeof(float), nq, out);
  fwrite(lse2, sizeof(float), (size_t)B * Hq * T, out);
  fwrite(o3, sizeof(float), nq, out);
  fwrite(lse3, sizeof(float), (size_t)B * Hq * T, out);
  fclose(out);
  hipStreamDestroy(stream);
  hipFree(d_parent); hipFree(d_off); hipFree(d_q); hipFree(d_kp); hipFree(d_vp);
  hipFree(d_kt); hipFree(d_vt); hipFree(d_mask); hipFree(d_status); hipFree(d_o);
  hipFree(d_lse); hipFree(d_ws); hipFree(d_kv); hipFree(d_o2); hipFree(d_lse2);
  hipFree(d_o3); hipFree(d_lse3); hipFree(d_ws3);
  free(parent); free(offsets); free(q); free(kp); free(vp); free(kt); free(vt); free(kv);
  free(mask); free(o); free(lse); free(o2); free(lse2); free(o3); free(lse3);
  return rc[0] == LTREE_OK && rc[1] == LTREE_OK && rc[2] == LTREE_OK && rc[3] == LTREE_OK ? 0 : 2;
}
