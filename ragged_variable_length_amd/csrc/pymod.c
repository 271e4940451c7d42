/*
 * pymod.c -- CPython extension `_rattn`: one function per rattn_* entry point
 * of include/rattn.h, taking plain Python ints (device pointers, sizes, enum
 * codes, the stream handle) and floats, and returning the rattn_status code.
 *
 * Argument marshalling only: every function converts its arguments and calls
 * the C entry point; there is no other code path.  It exists because a ctypes
 * call with fourteen converted arguments costs several microseconds of host
 * time, which is the same order as a whole pack -> attend -> unpack launch at
 * serving batch sizes; a METH_FASTCALL function costs a fraction of that.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>

#include "rattn.h"

/* None -> NULL, int -> pointer; returns 0 on success, -1 with an exception. */
static int as_ptr(PyObject *o, const void **out) {
    if (o == Py_None) {
        *out = NULL;
        return 0;
    }
    *out = PyLong_AsVoidPtr(o);
    return (*out == NULL && PyErr_Occurred()) ? -1 : 0;
}

static int as_int(PyObject *o, int *out) {
    long v = PyLong_AsLong(o);
    if (v == -1 && PyErr_Occurred()) return -1;
    if (v < INT32_MIN || v > INT32_MAX) {
        PyErr_SetString(PyExc_OverflowError, "argument does not fit in int32");
        return -1;
    }
    *out = (int)v;
    return 0;
}

static int nargs_is(Py_ssize_t nargs, Py_ssize_t want, const char *fn) {
    if (nargs == want) return 0;
    PyErr_Format(PyExc_TypeError, "%s takes %zd arguments (%zd given)", fn, want, nargs);
    return -1;
}

#define PTR(i, name)                                           \
    const void *name;                                          \
    if (as_ptr(args[i], &name)) return NULL
#define INT(i, name)                                           \
    int name;                                                  \
    if (as_int(args[i], &name)) return NULL

static PyObject *py_init(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    (void)self;
    (void)args;
    if (nargs_is(nargs, 0, "init")) return NULL;
    return PyLong_FromLong(rattn_init());
}

static PyObject *py_status_string(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    (void)self;
    if (nargs_is(nargs, 1, "status_string")) return NULL;
    INT(0, s);
    return PyUnicode_FromString(rattn_status_string((rattn_status)s));
}

static PyObject *py_version(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    (void)self;
    (void)args;
    if (nargs_is(nargs, 0, "version")) return NULL;
    return PyLong_FromLong(rattn_version());
}

static PyObject *py_set_validate(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    (void)self;
    if (nargs_is(nargs, 1, "set_validate")) return NULL;
    INT(0, on);
    return PyLong_FromLong(rattn_set_validate(on));
}

static PyObject *py_get_validate(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    (void)self;
    (void)args;
    if (nargs_is(nargs, 0, "get_validate")) return NULL;
    return PyLong_FromLong(rattn_get_validate());
}

/* pack(srcs: sequence of int, dsts: sequence of int, keep, B, N, row_elems,
 *      dtype, cu_seqlens, max_seqlen_out|None, total_out|None, stream) */
static PyObject *py_pack(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    (void)self;
    if (nargs_is(nargs, 11, "pack")) return NULL;
    const void *src[RATTN_MAX_TENSORS] = {0}, *dst[RATTN_MAX_TENSORS] = {0};
    PyObject *seqs[2] = {args[0], args[1]};
    const void **outs[2] = {src, dst};
    Py_ssize_t n = -1;
    for (int s = 0; s < 2; ++s) {
        PyObject *fast = PySequence_Fast(seqs[s], "pack: srcs and dsts must be sequences");
        if (!fast) return NULL;
        const Py_ssize_t len = PySequence_Fast_GET_SIZE(fast);
        if (len < 1 || len > RATTN_MAX_TENSORS || (n >= 0 && len != n)) {
            Py_DECREF(fast);
            PyErr_SetString(PyExc_ValueError, "pack: 1-3 sources and as many destinations");
            return NULL;
        }
        n = len;
        for (Py_ssize_t i = 0; i < len; ++i) {
            if (as_ptr(PySequence_Fast_GET_ITEM(fast, i), &outs[s][i])) {
                Py_DECREF(fast);
                return NULL;
            }
        }
        Py_DECREF(fast);
    }
    PTR(2, keep);
    INT(3, B);
    INT(4, N);
    INT(5, row_elems);
    INT(6, dt);
    PTR(7, cu);
    PTR(8, mx);
    PTR(9, tot);
    PTR(10, stream);
    return PyLong_FromLong(rattn_pack((const void *const *)src, (void *const *)dst, (int)n,
                                      (const uint8_t *)keep, B, N, row_elems, (rattn_dtype)dt,
                                      (int32_t *)cu, (int32_t *)mx, (int32_t *)tot,
                                      (void *)stream));
}

/* forward(q, k, v, o, cu_seqlens, B, max_seqlen, H, head_dim, scale, dtype, stream) */
static PyObject *py_forward(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    (void)self;
    if (nargs_is(nargs, 12, "forward")) return NULL;
    PTR(0, q);
    PTR(1, k);
    PTR(2, v);
    PTR(3, o);
    PTR(4, cu);
    INT(5, B);
    INT(6, max_seqlen);
    INT(7, H);
    INT(8, head_dim);
    const double scale = PyFloat_AsDouble(args[9]);
    if (scale == -1.0 && PyErr_Occurred()) return NULL;
    INT(10, dt);
    PTR(11, stream);
    return PyLong_FromLong(rattn_forward(q, k, v, (void *)o, (const int32_t *)cu, B, max_seqlen,
                                         H, head_dim, (float)scale, (rattn_dtype)dt,
                                         (void *)stream));
}

/* unpack(src, dst_padded|None, cls|None, keep, cu_seqlens, B, N, row_elems, dtype, stream) */
static PyObject *py_unpack(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    (void)self;
    if (nargs_is(nargs, 10, "unpack")) return NULL;
    PTR(0, src);
    PTR(1, dst);
    PTR(2, cls);
    PTR(3, keep);
    PTR(4, cu);
    INT(5, B);
    INT(6, N);
    INT(7, row_elems);
    INT(8, dt);
    PTR(9, stream);
    return PyLong_FromLong(rattn_unpack(src, (void *)dst, (void *)cls, (const uint8_t *)keep,
                                        (const int32_t *)cu, B, N, row_elems, (rattn_dtype)dt,
                                        (void *)stream));
}

/* fused(q, k, v, keep, out_padded|None, cls|None, B, N, H, head_dim, max_seqlen, scale,
 *       dtype, stream) */
static PyObject *py_fused(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    (void)self;
    if (nargs_is(nargs, 14, "fused")) return NULL;
    PTR(0, q);
    PTR(1, k);
    PTR(2, v);
    PTR(3, keep);
    PTR(4, out);
    PTR(5, cls);
    INT(6, B);
    INT(7, N);
    INT(8, H);
    INT(9, head_dim);
    INT(10, max_seqlen);
    const double scale = PyFloat_AsDouble(args[11]);
    if (scale == -1.0 && PyErr_Occurred()) return NULL;
    INT(12, dt);
    PTR(13, stream);
    return PyLong_FromLong(rattn_fused(q, k, v, (const uint8_t *)keep, (void *)out, (void *)cls,
                                       B, N, H, head_dim, max_seqlen, (float)scale,
                                       (rattn_dtype)dt, (void *)stream));
}

/* fused_padded(q, k, v, keep, out_padded|None, cls|None, B, N, H, head_dim, pad_len, scale,
 *              dtype, stream) */
static PyObject *py_fused_padded(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    (void)self;
    if (nargs_is(nargs, 14, "fused_padded")) return NULL;
    PTR(0, q);
    PTR(1, k);
    PTR(2, v);
    PTR(3, keep);
    PTR(4, out);
    PTR(5, cls);
    INT(6, B);
    INT(7, N);
    INT(8, H);
    INT(9, head_dim);
    INT(10, pad_len);
    const double scale = PyFloat_AsDouble(args[11]);
    if (scale == -1.0 && PyErr_Occurred()) return NULL;
    INT(12, dt);
    PTR(13, stream);
    return PyLong_FromLong(rattn_fused_padded(q, k, v, (const uint8_t *)keep, (void *)out,
                                              (void *)cls, B, N, H, head_dim, pad_len,
                                              (float)scale, (rattn_dtype)dt, (void *)stream));
}

/* repack(srcs: sequence of int, dsts: sequence of int, keep2, cu_seqlens, B, row_elems, dtype,
 *        cu_seqlens_out, total_out|None, stream) */
static PyObject *py_repack(PyObject *self, PyObject *const *args, Py_ssize_t nargs) {
    (void)self;
    if (nargs_is(nargs, 10, "repack")) return NULL;
    const void *src[RATTN_MAX_TENSORS] = {0}, *dst[RATTN_MAX_TENSORS] = {0};
    PyObject *seqs[2] = {args[0], args[1]};
    const void **outs[2] = {src, dst};
    Py_ssize_t n = -1;
    for (int s = 0; s < 2; ++s) {
        PyObject *fast = PySequence_Fast(seqs[s], "repack: srcs and dsts must be sequences");
        if (!fast) return NULL;
        const Py_ssize_t len = PySequence_Fast_GET_SIZE(fast);
        if (len < 1 || len > RATTN_MAX_TENSORS || (n >= 0 && len != n)) {
            Py_DECREF(fast);
            PyErr_SetString(PyExc_ValueError, "repack: 1-3 sources and as many destinations");
            return NULL;
        }
        n = len;
        for (Py_ssize_t i = 0; i < len; ++i) {
            if (as_ptr(PySequence_Fast_GET_ITEM(fast, i), &outs[s][i])) {
                Py_DECREF(fast);
                return NULL;
            }
        }
        Py_DECREF(fast);
    }
    PTR(2, keep2);
    PTR(3, cu);
    INT(4, B);
    INT(5, row_elems);
    INT(6, dt);
    PTR(7, cu2);
    PTR(8, tot);
    PTR(9, stream);
    return PyLong_FromLong(rattn_repack((const void *const *)src, (void *const *)dst, (int)n,
                                        (const uint8_t *)keep2, (const int32_t *)cu, B, row_elems,
                                        (rattn_dtype)dt, (int32_t *)cu2, (int32_t *)tot,
                                        (void *)stream));
}

static PyMethodDef methods[] = {
    {"init", (PyCFunction)(void (*)(void))py_init, METH_FASTCALL, "rattn_init()"},
    {"status_string", (PyCFunction)(void (*)(void))py_status_string, METH_FASTCALL,
     "rattn_status_string(status)"},
    {"version", (PyCFunction)(void (*)(void))py_version, METH_FASTCALL, "rattn_version()"},
    {"set_validate", (PyCFunction)(void (*)(void))py_set_validate, METH_FASTCALL,
     "rattn_set_validate(on)"},
    {"get_validate", (PyCFunction)(void (*)(void))py_get_validate, METH_FASTCALL,
     "rattn_get_validate()"},
    {"pack", (PyCFunction)(void (*)(void))py_pack, METH_FASTCALL, "rattn_pack(...)"},
    {"forward", (PyCFunction)(void (*)(void))py_forward, METH_FASTCALL, "rattn_forward(...)"},
    {"unpack", (PyCFunction)(void (*)(void))py_unpack, METH_FASTCALL, "rattn_unpack(...)"},
    {"fused", (PyCFunction)(void (*)(void))py_fused, METH_FASTCALL, "rattn_fused(...)"},
    {"fused_padded", (PyCFunction)(void (*)(void))py_fused_padded, METH_FASTCALL,
     "rattn_fused_padded(...)"},
    {"repack", (PyCFunction)(void (*)(void))py_repack, METH_FASTCALL, "rattn_repack(...)"},
    {NULL, NULL, 0, NULL}};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_rattn",
                                    "Argument marshalling for librattn.so's C entry points.",
                                    -1, methods, NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__rattn(void) { return PyModule_Create(&module); }
