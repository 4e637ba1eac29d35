// paged.hip -- the paged optimizer: AdamW on LoRA tensors whose moment
// estimates live in a pinned host backing store and are paged through a
// device working buffer of the caller's size.
//
// glossary "QLoRA", Definition: paged optimizers manage memory spikes;
// deepfa.ir blog, "3. Paged Optimizers": optimizer states move between GPU
// and CPU memory as needed.  The policy, decided per call from the sizes
// alone (so every call with the same tensors and budget makes the same
// choice):
//   - everything fits the budget: every tensor's moments are resident in the
//     device buffer;
//   - otherwise two staging slots of `chunk` values (m and v each) are carved
//     first, and the leading tensors whose moments fit the rest are resident;
//     the other tensors are paged: each chunk is copied host -> device on the
//     copy stream into a free slot, updated on the compute stream, and copied
//     back, the copy of chunk i+1 overlapping the update of chunk i (events
//     order the two streams).
// Resident moments stay in the device buffer between calls: the caller loads
// them from the backing store once (QLORA_PAGED_LOAD) and stores them back
// when it needs the host copy (QLORA_PAGED_STORE), for example to checkpoint.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "../../include/qlora.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr size_t kPagedAlign = 256;
constexpr int64_t kMaxChunk = (int64_t)4 << 20;   // values per staging slot at most (32 MiB of m and v)
constexpr int64_t kChunkQuantum = 64;             // chunks are whole multiples of 64 values

size_t pal(size_t x) { return (x + kPagedAlign - 1) / kPagedAlign * kPagedAlign; }
size_t state_bytes(int64_t n) { return 2 * pal((size_t)n * sizeof(float)); }   // m then v

}  // namespace

// Layout of the device buffer: [slot 0: m | v][slot 1: m | v][resident
// tensor 0: m | v][resident tensor 1: m | v] ..., every piece 256-aligned.
bool paged_plan(const qlora_paged_tensor* t, int nt, size_t dev_bytes, qlora_paged_layout* L) {
  size_t total = 0;
  for (int i = 0; i < nt; ++i) total += state_bytes(t[i].n);
  L->chunk = 0;
  L->staging_bytes = 0;
  if (total <= dev_bytes) {
    L->resident = nt;
    L->resident_bytes = total;
    return true;
  }
  int64_t chunk = std::min<int64_t>(kMaxChunk, (int64_t)(dev_bytes / 4 / (2 * sizeof(float))));
  chunk = chunk / kChunkQuantum * kChunkQuantum;
  if (chunk < kChunkQuantum) return false;   // not even two minimal slots
  L->chunk = (size_t)chunk;
  L->staging_bytes = 2 * state_bytes(chunk);
  size_t used = L->staging_bytes;
  int res = 0;
  while (res < nt && used + state_bytes(t[res].n) <= dev_bytes) used += state_bytes(t[res++].n);
  L->resident = res;
  L->resident_bytes = used - L->staging_bytes;
  return true;
}

hipError_t paged_adamw(const qlora_paged_tensor* t, int nt, char* ws, const qlora_paged_layout& L, float lr,
                       float b1, float b2, float eps, float wd, int step, int flags, hipStream_t st,
                       hipStream_t cp) {
  hipError_t e = hipSuccess;
  // resident tensors
  size_t off = L.staging_bytes;
  for (int i = 0; i < L.resident; ++i) {
    const int64_t n = t[i].n;
    float* m = reinterpret_cast<float*>(ws + off);
    float* v = reinterpret_cast<float*>(ws + off + pal((size_t)n * sizeof(float)));
    const size_t nb = (size_t)n * sizeof(float);
    if (flags & QLORA_PAGED_LOAD) {
      if ((e = hipMemcpyAsync(m, t[i].m, nb, hipMemcpyHostToDevice, st)) != hipSuccess) return e;
      if ((e = hipMemcpyAsync(v, t[i].v, nb, hipMemcpyHostToDevice, st)) != hipSuccess) return e;
    }
    if ((e = launch_adamw(t[i].p, t[i].p_bf16, t[i].grad, m, v, n, lr, b1, b2, eps, wd, step, st)) != hipSuccess)
      return e;
    if (flags & QLORA_PAGED_STORE) {
      if ((e = hipMemcpyAsync(t[i].m, m, nb, hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
      if ((e = hipMemcpyAsync(t[i].v, v, nb, hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
    }
    off += state_bytes(n);
  }
  if (L.resident == nt) return hipSuccess;

  // paged tensors, chunk by chunk through the two staging slots
  struct Item {
    int t;
    int64_t off, len;
  };
  std::vector<Item> items;
  for (int i = L.resident; i < nt; ++i)
    for (int64_t o = 0; o < t[i].n; o += (int64_t)L.chunk)
      items.push_back(Item{i, o, std::min<int64_t>((int64_t)L.chunk, t[i].n - o)});
  float* sm[2];
  float* sv[2];
  for (int k = 0; k < 2; ++k) {
    sm[k] = reinterpret_cast<float*>(ws + k * state_bytes((int64_t)L.chunk));
    sv[k] = reinterpret_cast<float*>(ws + k * state_bytes((int64_t)L.chunk) + pal(L.chunk * sizeof(float)));
  }
  const bool two = cp != nullptr && cp != st;
  hipStream_t cs = two ? cp : st;
  hipEvent_t ev[5] = {};   // loaded[2], updated[2], start / done
  auto destroy = [&]() {
    for (hipEvent_t x : ev)
      if (x) (void)hipEventDestroy(x);   // released once their last use has completed
  };
  if (two) {
    for (hipEvent_t& x : ev)
      if ((e = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess) {
        destroy();
        return e;
      }
    // the copies follow whatever the compute stream holds before this call
    if ((e = hipEventRecord(ev[4], st)) != hipSuccess || (e = hipStreamWaitEvent(cs, ev[4], 0)) != hipSuccess) {
      destroy();
      return e;
    }
  }
  auto copy_back = [&](size_t j) -> hipError_t {
    const Item& it = items[j];
    const int k = (int)(j & 1);
    hipError_t r = hipSuccess;
    if (two && (r = hipStreamWaitEvent(cs, ev[2 + k], 0)) != hipSuccess) return r;
    const size_t nb = (size_t)it.len * sizeof(float);
    if ((r = hipMemcpyAsync(t[it.t].m + it.off, sm[k], nb, hipMemcpyDeviceToHost, cs)) != hipSuccess) return r;
    return hipMemcpyAsync(t[it.t].v + it.off, sv[k], nb, hipMemcpyDeviceToHost, cs);
  };
  for (size_t j = 0; j < items.size(); ++j) {
    const Item& it = items[j];
    const int k = (int)(j & 1);
    // the slot's previous chunk goes back to the host first (same copy stream)
    if (j >= 2 && (e = copy_back(j - 2)) != hipSuccess) break;
    const size_t nb = (size_t)it.len * sizeof(float);
    if ((e = hipMemcpyAsync(sm[k], t[it.t].m + it.off, nb, hipMemcpyHostToDevice, cs)) != hipSuccess) break;
    if ((e = hipMemcpyAsync(sv[k], t[it.t].v + it.off, nb, hipMemcpyHostToDevice, cs)) != hipSuccess) break;
    if (two && ((e = hipEventRecord(ev[k], cs)) != hipSuccess || (e = hipStreamWaitEvent(st, ev[k], 0)) != hipSuccess))
      break;
    const qlora_paged_tensor& T = t[it.t];
    if ((e = launch_adamw(T.p + it.off, T.p_bf16 ? T.p_bf16 + it.off : nullptr, T.grad + it.off, sm[k], sv[k], it.len,
                          lr, b1, b2, eps, wd, step, st)) != hipSuccess)
      break;
    if (two && (e = hipEventRecord(ev[2 + k], st)) != hipSuccess) break;
  }
  for (size_t j = items.size() >= 2 ? items.size() - 2 : 0; e == hipSuccess && j < items.size(); ++j)
    e = copy_back(j);
  // the compute stream is done only when the last copy back is
  if (e == hipSuccess && two && (e = hipEventRecord(ev[4], cs)) == hipSuccess) e = hipStreamWaitEvent(st, ev[4], 0);
  destroy();
  return e;
}

}  // namespace qlora
