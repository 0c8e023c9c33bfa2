// kv_pages.h -- device addressing of the paged KV cache (internal).
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace dflash {

// V pages store the positions of every 32-slot group in the order
//   0-3, 16-19, 4-7, 20-23, 8-11, 24-27, 12-15, 28-31
// so that the 8 positions one lane feeds to a 32-key P.V matrix-core step
// (4 from each 16-key half) are 8 consecutive elements.
__host__ __device__ __forceinline__ int vslot(int slot) {
    const int k = slot & 31;
    const int pos = k < 16 ? 8 * (k >> 2) + (k & 3) : 8 * ((k - 16) >> 2) + 4 + (k & 3);
    return (slot & ~31) | pos;
}

// Paged draft-KV addressing: per (layer, K|V) an array of pages; K pages are
// [nkv][page][d] (key rows), V pages [nkv][d][page] (value columns, so the
// attention's P.V operand reads runs of consecutive positions).
struct KVPages {
    char* base;
    const int32_t* table;
    long long layer_kv_bytes;  // bytes of one (layer, K|V) page array
    int page, nkv, d, elem;
    __device__ __forceinline__ long long page_elems() const { return (long long)nkv * page * d; }
    template <typename T>
    __device__ __forceinline__ T* kpage(int l, int pos, int& slot) const {
        const int p = pos / page;
        slot = pos - p * page;
        return reinterpret_cast<T*>(base + (2LL * l) * layer_kv_bytes) + (long long)table[p] * page_elems();
    }
    template <typename T>
    __device__ __forceinline__ T* vpage(int l, int pos, int& slot) const {
        const int p = pos / page;
        slot = pos - p * page;
        return reinterpret_cast<T*>(base + (2LL * l + 1) * layer_kv_bytes) + (long long)table[p] * page_elems();
    }
    // the same, for an already looked-up physical page
    template <typename T>
    __device__ __forceinline__ T* kpage_phys(int l, int phys) const {
        return reinterpret_cast<T*>(base + (2LL * l) * layer_kv_bytes) + (long long)phys * page_elems();
    }
    template <typename T>
    __device__ __forceinline__ T* vpage_phys(int l, int phys) const {
        return reinterpret_cast<T*>(base + (2LL * l + 1) * layer_kv_bytes) + (long long)phys * page_elems();
    }
};

template <typename T>
static inline KVPages make_pages(const DevCtx& c) {
    KVPages kv;
    kv.base = c.kv;
    kv.table = reinterpret_cast<const int32_t*>(c.ws + c.lay.page_table);
    kv.layer_kv_bytes = (long long)c.lay.kv_layer_kv;
    kv.page = c.dm.page;
    kv.nkv = c.dm.nkv;
    kv.d = c.dm.d;
    kv.elem = c.dm.elem;
    return kv;
}

}  // namespace dflash
